// gfx950 kernel of the decode-batch attention front.
//
// The projection y = x W^T for M <= 16 tokens is a weight stream: every
// element of W (up to 151 MB) is read once and meets at most 16 token values,
// so the call is bound by HBM bandwidth, not by the matrix cores.  One kernel
// does the whole call:
//
//  Projection: 256 blocks (one per CU, all resident together) of 8 waves.
//    Block b owns a contiguous K range of 8192/S (S = 32/nkv splits) and 9
//    row tiles of 16 W rows.  For each tile the block
//      - loads the 16 rows with non-temporal 16-byte loads, each wave
//        instruction reading 1 KB of one row (the shape HBM streams best),
//        several tiles ahead of use, into registers;
//      - stores them into an LDS tile whose 16-byte chunks are XOR-swizzled
//        by row, so the transposed reads below hit distinct banks;
//      - reads the tile back in MFMA operand layout, each wave its own 1/8 of
//        the block's K range, and issues v_mfma_f32_16x16x32_bf16 with W as
//        the 16-row A operand and the tokens (x, held in registers for the
//        whole kernel, zero past M) as the 16 B columns.
//    The 8 wave partials of each tile are summed in LDS in wave order and
//    the block's fp32 partial goes to the workspace, each value stored
//    together with the number of the call in one 64-bit word.
//
//  Epilogue: each (pair of heads, token) is one item of one wave.  The wave
//    fetched its token's slot and cos|sin row while the weights streamed; it
//    reads the S partials of each of its columns until all carry this call's
//    number (a bounded wait), sums them in
//    split order, rounds to bf16 (round to nearest even), applies to q and k
//    heads the weightless RMS norm (sum of squares by a butterfly of lane
//    exchanges) and the interleaved rotation, and stores its part of y and of
//    the token's K|V slot.
//
//  No read-modify-write atomics, no flags to wait for and no cache
//  maintenance: each partial travels with its call number in one 64-bit
//  device-coherent (agent-scope) store, and a reader accepts a value only
//  when its tag is the current call's.  The call number comes from a
//  per-block counter that every call raises by one (so all counters agree at
//  the start of a call, and a graph replay gets a new number).  The sums run
//  in a fixed order, so the result depends on the launch shape only.
//
// Definitions followed: qkv_front page, module summary (projection, norm,
// RoPE, y store, K/V insert) and "Structure" (partials summed in a fixed
// rank order by the owner, rounded to bf16, then the epilogue; the aux warp
// that fetches slots and cos|sin rows); cute_ops page, split_qkv (column
// blocks) and the attn2 contract (cache layout).
#include <hip/hip_runtime.h>

#include "qkvf_internal.h"

namespace qkvf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kEps = 1e-6f;

template <int NKV>
struct Shape {
    static constexpr int N = cols_for(NKV);
    static constexpr int S = splits_for(NKV);      // K splits across blocks
    static constexpr int KB = kHidden / S;         // K per block: 256 * NKV
    static constexpr int KW = KB / kWaves;         // K per wave: 32 * NKV
    static constexpr int STEPS = KW / 32;          // MFMA K steps per tile and wave
    static constexpr int GROUPS = kGrid / S;       // row groups of 9 tiles
    static constexpr int CHUNKS = KB / 8;          // 16-byte chunks per tile row
    static constexpr int LOADS = 2 * CHUNKS / 64;  // 1 KB loads per wave per tile (2 rows)
    static constexpr int TILE_BYTES = kTileRows * KB * 2;
    // The wave partials of all tiles, summed at the end, reuse the same LDS.
    static constexpr int RED_BYTES = 4 * kWaves * kTilesPerBlock * kTileRows * (kTileRows + 1);
    static constexpr int LDS_BYTES = 2 * TILE_BYTES > RED_BYTES ? 2 * TILE_BYTES : RED_BYTES;
    // Tiles of loads in flight per wave: up to 12 loads of 1 KB per wave.
    static constexpr int DEPTH = (12 / LOADS) < kTilesPerBlock ? (12 / LOADS) : kTilesPerBlock;
    static_assert(S * GROUPS == kGrid, "grid covers every (split, group)");
    static_assert(GROUPS * kTilesPerBlock * kTileRows == N, "groups cover N");
    static_assert(KW % 32 == 0 && CHUNKS % 16 == 0, "whole MFMA steps, whole swizzle groups");
    static_assert(LOADS * 64 == 2 * CHUNKS, "each wave loads exactly two tile rows");
};

__device__ inline bf16x8 load16(const __bf16 *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

// W is read once: non-temporal loads keep it from displacing reused lines.
__device__ inline bf16x8 stream16(const __bf16 *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
}

__device__ inline unsigned pack2(__bf16 lo, __bf16 hi)
{
    return unsigned(__builtin_bit_cast(unsigned short, lo)) |
           (unsigned(__builtin_bit_cast(unsigned short, hi)) << 16);
}

template <int NKV>
__global__ void __launch_bounds__(kWaves * 64, 1)
front_fused(const __bf16 *__restrict__ x, const __bf16 *__restrict__ W,
            const int64_t *__restrict__ positions, const int64_t *__restrict__ slots,
            const float *__restrict__ cos_sin, __bf16 *__restrict__ y,
            __bf16 *__restrict__ kv_cache, float *__restrict__ ws, int M)
{
    using Sh = Shape<NKV>;
    constexpr int ST = Sh::STEPS, D = Sh::DEPTH, U = kTilesPerBlock, C = Sh::CHUNKS;
    constexpr int LD = Sh::LOADS, N = Sh::N, NQ = kQPerKv * NKV;
    constexpr int PAIRS = N / (2 * kHeadDim);  // epilogue items per token
    constexpr size_t kTileStride = size_t(kTileRows) * kHidden;
    __shared__ __attribute__((aligned(16))) unsigned char lds[Sh::LDS_BYTES];

    unsigned *words = reinterpret_cast<unsigned *>(ws);
    unsigned *ready = words + kReadyOffset;
    uint64_t *parts = reinterpret_cast<uint64_t *>(ws);
    const int b = blockIdx.x;
    // Every call raises every block's flag by one, so at the start of a call
    // all flags hold the number of calls made so far; this call's value is
    // one more.  A block reads only its own flag, written by itself in the
    // previous call.
    const unsigned target =
        __hip_atomic_load(ready + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
    const int split = b % Sh::S;
    const int group = b / Sh::S;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;   // A row (W row in the tile) and B column (token)
    const int q = lane >> 4;   // which 8 of the 32 K values of a step
    const int k0 = split * Sh::KB;

    // This wave's epilogue item, if any: head pair `pair` of token `tok`.
    const int item = wave * kGrid + b;
    const bool has_item = item < PAIRS * M;
    const int tok = has_item ? item / PAIRS : 0;
    const int pair = item - tok * PAIRS;
    const int pi = lane & 31;  // rotation pair within the lane's head
    // Unconditional loads (tok < M always), so nothing waits on them until
    // they are used.
    const int64_t pos_t = positions[tok];
    const int64_t slot_t = slots[tok];

    // Chunk (8 K values) of this lane's operands in MFMA step st, relative to
    // k0: A (W) and B (x) use the same chunk, so the MFMA contracts matching
    // K values.
    auto chunk_of = [&](int st) { return wave * 4 * ST + st * 4 + q; };

    // Token columns r >= M repeat row M-1; their MFMA outputs are never used.
    const int xrow = r < M ? r : M - 1;
    bf16x8 xv[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st)
        xv[st] = load16(x + size_t(xrow) * kHidden + k0 + chunk_of(st) * 8);

    // Load j of this wave covers chunk c of tile row `row` (rows 2w, 2w+1);
    // it lands in LDS chunk row * C + (c ^ row).
    const __bf16 *wtile = W + size_t(group * U * kTileRows) * kHidden + k0;
    size_t goff[LD];
    int loff[LD];
#pragma unroll
    for (int j = 0; j < LD; ++j) {
        const int L = j * 64 + lane;
        const int row = 2 * wave + L / C;
        const int c = L % C;
        goff[j] = size_t(row) * kHidden + c * 8;
        loff[j] = (row * C + (c ^ (row & 15))) * 16;
    }

    bf16x8 ring[D][LD];
#pragma unroll
    for (int u = 0; u < D; ++u)
#pragma unroll
        for (int j = 0; j < LD; ++j)
            ring[u][j] = stream16(wtile + u * kTileStride + goff[j]);

    // The token's rotation for this lane's pair, fetched while W streams.
    // The barriers keep this dependent load behind the weight prologue, so
    // waiting for the position never stalls the stream.
    __builtin_amdgcn_sched_barrier(0);
    const float *cs_row = cos_sin != nullptr ? cos_sin + pos_t * kHeadDim
                                             : reinterpret_cast<const float *>(ws);
    float rc = cs_row[pi], rs = cs_row[32 + pi];
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        unsigned char *tile = lds + (u & 1) * Sh::TILE_BYTES;
#pragma unroll
        for (int j = 0; j < LD; ++j)
            *reinterpret_cast<bf16x8 *>(tile + loff[j]) = ring[u % D][j];
        if (u + D < U) {
#pragma unroll
            for (int j = 0; j < LD; ++j)
                ring[u % D][j] = stream16(wtile + (u + D) * kTileStride + goff[j]);
        }
        __syncthreads();
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int c = chunk_of(st);
            const bf16x8 w = *reinterpret_cast<const bf16x8 *>(tile + (r * C + (c ^ r)) * 16);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xv[st], a, 0, 0, 0);
        }
        acc[u] = a;
    }

    // Lane (r, q) holds D[row = 4q + v][token = r], v = 0..3.  Sum the 8
    // waves' partials of every tile in wave order through LDS (reusing the
    // tile buffers) and write the block's partial ws[split][token][n].
    float(*red)[U][kTileRows][kTileRows + 1] =
        reinterpret_cast<float(*)[U][kTileRows][kTileRows + 1]>(lds);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[wave][u][r][4 * q + v] = acc[u][v];
    __syncthreads();
    const int per_tile = kTileRows * M;
    for (int e = threadIdx.x; e < U * per_tile; e += kWaves * 64) {
        const int u = e / per_tile;
        const int rem = e - u * per_tile;
        const int t = rem >> 4, row = rem & 15;
        float sum = red[0][u][t][row];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            sum += red[w][u][t][row];
        const int n = (group * U + u) * kTileRows + row;
        __hip_atomic_store(parts + (size_t(split) * M + t) * N + n,
                           (uint64_t(target) << 32) | __float_as_uint(sum), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }

    // Count this call in the block's flag (read back at the next call's start).
    if (threadIdx.x == 0)
        __hip_atomic_store(ready + b, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    if (has_item) {
        // The S partials of this lane's two columns, each tagged with the
        // call that wrote it: poll (bounded) until every tag is this call's,
        // then sum in split order.
        const int h = 2 * pair + (lane >> 5);  // head of this half-wave
        const int n = h * kHeadDim + 2 * pi;
        const uint64_t *src = parts + size_t(tok) * N + n;
        constexpr size_t kSplitStride = size_t(N);  // times M, below
        uint64_t v[Sh::S][2];
        for (unsigned tries = 0;; ++tries) {
            bool mine = true;
#pragma unroll
            for (int s = 0; s < Sh::S; ++s)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    v[s][c] = __hip_atomic_load(src + size_t(s) * M * kSplitStride + c,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    mine = mine && unsigned(v[s][c] >> 32) == target;
                }
            if (__all(mine))
                break;
            if (tries >= kSpinLimit) {
                words[kFaultWord] = kFaultTimeout;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int s = 0; s < Sh::S; ++s) {
            a0 += __uint_as_float(unsigned(v[s][0]));
            a1 += __uint_as_float(unsigned(v[s][1]));
        }
        const __bf16 p0 = __bf16(a0), p1 = __bf16(a1);
        const float f0 = float(p0), f1 = float(p1);

        // Sum of squares of the head's 64 values: butterfly over the 32 lanes
        // of the half-wave (every lane ends with the same total).
        float ss = f0 * f0 + f1 * f1;
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1)
            ss += __shfl_xor(ss, m, 64);

        if (cos_sin == nullptr) {  // a layer without RoPE: norm only
            rc = 1.f;
            rs = 0.f;
        }
        __bf16 o0 = p0, o1 = p1;
        if (h < NQ + NKV) {  // q and k heads
            const float rr = rsqrtf(ss * (1.0f / kHeadDim) + kEps);
            const float n0 = f0 * rr, n1 = f1 * rr;
            o0 = __bf16(n0 * rc - n1 * rs);
            o1 = __bf16(n1 * rc + n0 * rs);
        }
        const unsigned packed = pack2(o0, o1);
        *reinterpret_cast<unsigned *>(y + size_t(tok) * N + n) = packed;

        if (slot_t >= 0 && h >= NQ && h < NQ + 2 * NKV) {
            const int64_t page = slot_t / kPageSlots, off = slot_t % kPageSlots;
            const bool is_k = h < NQ + NKV;
            const int j = is_k ? h - NQ : h - NQ - NKV;
            __bf16 *dst = kv_cache + ((page * NKV + j) * kPageSlots + off) * kSlotWidth +
                          (is_k ? 0 : kHeadDim) + 2 * pi;
            *reinterpret_cast<unsigned *>(dst) = packed;
        }
    }

}

template <int NKV>
hipError_t launch(int M, const void *x, const void *W, const int64_t *positions,
                  const int64_t *slots, const float *cos_sin, void *y, void *kv_cache,
                  float *ws, hipStream_t stream)
{
    hipLaunchKernelGGL(front_fused<NKV>, dim3(kGrid), dim3(kWaves * 64), 0, stream,
                       static_cast<const __bf16 *>(x), static_cast<const __bf16 *>(W),
                       positions, slots, cos_sin, static_cast<__bf16 *>(y),
                       static_cast<__bf16 *>(kv_cache), ws, M);
    return hipGetLastError();
}

template <int NKV>
int occupancy()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, front_fused<NKV>, kWaves * 64, 0) !=
        hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

}  // namespace

hipError_t launch_front(int nkv, int M, const void *x, const void *W,
                        const int64_t *positions, const int64_t *slots,
                        const float *cos_sin, void *y, void *kv_cache, float *ws,
                        hipStream_t stream)
{
    switch (nkv) {
    case 1: return launch<1>(M, x, W, positions, slots, cos_sin, y, kv_cache, ws, stream);
    case 2: return launch<2>(M, x, W, positions, slots, cos_sin, y, kv_cache, ws, stream);
    case 4: return launch<4>(M, x, W, positions, slots, cos_sin, y, kv_cache, ws, stream);
    case 8: return launch<8>(M, x, W, positions, slots, cos_sin, y, kv_cache, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

int blocks_per_cu(int nkv)
{
    switch (nkv) {
    case 1: return occupancy<1>();
    case 2: return occupancy<2>();
    case 4: return occupancy<4>();
    case 8: return occupancy<8>();
    default: return 0;
    }
}

}  // namespace qkvf
