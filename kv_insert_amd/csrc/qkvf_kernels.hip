// gfx950 kernels of the decode-batch attention front.
//
// The projection y = x W^T for M <= 16 tokens is a weight stream: every
// element of W (up to 151 MB) is read once and meets at most 16 token values,
// so the call is bound by HBM bandwidth, not by the matrix cores.  Two
// kernels run back to back on the caller's stream:
//
//  front_partials: 256 blocks (one per CU) of 8 waves.  Block b owns a
//    contiguous K range of 8192/S (S = 32/nkv splits) and 9 row tiles of 16
//    W rows.  For each tile the block
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
//    the block's fp32 partial goes to the workspace: no atomics, fixed order.
//    Blocks 0..M-1 also gather their token's cos|sin row and slot into the
//    workspace, so the epilogue has no dependent loads.
//
//  front_epilogue: one wave per (token, 2 heads).  Sums the S partials of
//    each column in split order, rounds to bf16 (round to nearest even), and
//    for q and k heads applies the weightless RMS norm (sum of squares by a
//    butterfly of lane exchanges) and the interleaved rotation; stores the
//    row of y and the token's K|V slot.
//
// Definitions followed: qkv_front page, module summary (projection, norm,
// RoPE, y store, K/V insert) and "Structure" (partials summed in a fixed
// rank order, rounded to bf16, then the epilogue; the aux warp that fetches
// slots and cos|sin rows); cute_ops page, split_qkv (column blocks) and the
// attn2 contract (cache layout).
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
    // Tiles of loads in flight per wave: about 24 loads (96 VGPRs).
    static constexpr int DEPTH = (24 / LOADS) < kTilesPerBlock ? (24 / LOADS) : kTilesPerBlock;
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

template <int NKV>
__global__ void __launch_bounds__(kWaves * 64, 1)
front_partials(const __bf16 *__restrict__ x, const __bf16 *__restrict__ W,
               const int64_t *__restrict__ positions, const int64_t *__restrict__ slots,
               const float *__restrict__ cos_sin, float *__restrict__ ws, int M)
{
    using Sh = Shape<NKV>;
    constexpr int ST = Sh::STEPS, D = Sh::DEPTH, U = kTilesPerBlock, C = Sh::CHUNKS;
    constexpr int LD = Sh::LOADS;
    constexpr size_t kTileStride = size_t(kTileRows) * kHidden;
    __shared__ __attribute__((aligned(16))) unsigned char lds[Sh::LDS_BYTES];

    const int b = blockIdx.x;
    const int split = b % Sh::S;
    const int group = b / Sh::S;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;   // A row (W row in the tile) and B column (token)
    const int q = lane >> 4;   // which 8 of the 32 K values of a step
    const int k0 = split * Sh::KB;

    // Blocks 0..M-1 fetch their token's cos|sin row and slot for the
    // epilogue before the weight stream starts.
    if (b < M && wave == 0) {
        float *aux_rows = ws + kAuxRowsOffset;
        if (cos_sin != nullptr)
            aux_rows[b * kHeadDim + lane] = cos_sin[positions[b] * kHeadDim + lane];
        if (lane == 0)
            reinterpret_cast<int64_t *>(ws + kAuxSlotsOffset)[b] = slots[b];
    }

    // Chunk (8 K values) of this lane's operands in MFMA step st, relative to
    // k0: A (W) and B (x) use the same chunk, so the MFMA contracts matching
    // K values.
    auto chunk_of = [&](int st) { return wave * 4 * ST + st * 4 + q; };

    bf16x8 xv[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
        if (r < M)
            xv[st] = load16(x + size_t(r) * kHidden + k0 + chunk_of(st) * 8);
        else
            xv[st] = bf16x8{};
    }

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
        const int tok = rem >> 4, row = rem & 15;
        float sum = red[0][u][tok][row];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            sum += red[w][u][tok][row];
        const int n = (group * U + u) * kTileRows + row;
        ws[(size_t(split) * M + tok) * Sh::N + n] = sum;
    }
}

__device__ inline unsigned pack2(__bf16 lo, __bf16 hi)
{
    return unsigned(__builtin_bit_cast(unsigned short, lo)) |
           (unsigned(__builtin_bit_cast(unsigned short, hi)) << 16);
}

template <int NKV>
__global__ void __launch_bounds__(64)
front_epilogue(const float *__restrict__ ws, bool rope, __bf16 *__restrict__ y,
               __bf16 *__restrict__ kv_cache, int M)
{
    using Sh = Shape<NKV>;
    constexpr int N = Sh::N, NQ = kQPerKv * NKV;
    const int t = blockIdx.y;
    const int lane = threadIdx.x;
    const int h = 2 * blockIdx.x + (lane >> 5);  // head of this half-wave
    const int i = lane & 31;                      // rotation pair of the head
    const int n = h * kHeadDim + 2 * i;

    const float *row = ws + kAuxRowsOffset + t * kHeadDim;
    const float c = rope ? row[i] : 1.f;
    const float sn = rope ? row[32 + i] : 0.f;
    const int64_t slot = reinterpret_cast<const int64_t *>(ws + kAuxSlotsOffset)[t];

    float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
    for (int s = 0; s < Sh::S; ++s) {
        const float2 v = *reinterpret_cast<const float2 *>(ws + (size_t(s) * M + t) * N + n);
        a0 += v.x;
        a1 += v.y;
    }
    const __bf16 p0 = __bf16(a0), p1 = __bf16(a1);
    const float f0 = float(p0), f1 = float(p1);

    // Sum of squares of the head's 64 values: butterfly over the 32 lanes of
    // the half-wave (every lane ends with the same total).
    float ss = f0 * f0 + f1 * f1;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1)
        ss += __shfl_xor(ss, m, 64);

    const bool normed = h < NQ + NKV;  // q and k heads
    __bf16 o0 = p0, o1 = p1;
    if (normed) {
        const float rr = rsqrtf(ss * (1.0f / kHeadDim) + kEps);
        const float n0 = f0 * rr, n1 = f1 * rr;
        if (rope) {
            o0 = __bf16(n0 * c - n1 * sn);
            o1 = __bf16(n1 * c + n0 * sn);
        } else {
            o0 = __bf16(n0);
            o1 = __bf16(n1);
        }
    }
    const unsigned packed = pack2(o0, o1);
    *reinterpret_cast<unsigned *>(y + size_t(t) * N + n) = packed;

    if (slot >= 0 && h >= NQ && h < NQ + 2 * NKV) {
        const int64_t page = slot / kPageSlots, off = slot % kPageSlots;
        const bool is_k = h < NQ + NKV;
        const int j = is_k ? h - NQ : h - NQ - NKV;
        __bf16 *dst = kv_cache + ((page * NKV + j) * kPageSlots + off) * kSlotWidth +
                      (is_k ? 0 : kHeadDim) + 2 * i;
        *reinterpret_cast<unsigned *>(dst) = packed;
    }
}

template <int NKV>
hipError_t launch(int M, const void *x, const void *W, const int64_t *positions,
                  const int64_t *slots, const float *cos_sin, void *y, void *kv_cache,
                  float *ws, hipStream_t stream)
{
    using Sh = Shape<NKV>;
    hipLaunchKernelGGL(front_partials<NKV>, dim3(kGrid), dim3(kWaves * 64), 0, stream,
                       static_cast<const __bf16 *>(x), static_cast<const __bf16 *>(W),
                       positions, slots, cos_sin, ws, M);
    hipLaunchKernelGGL(front_epilogue<NKV>, dim3(Sh::N / (2 * kHeadDim), M), dim3(64), 0,
                       stream, ws, cos_sin != nullptr, static_cast<__bf16 *>(y),
                       static_cast<__bf16 *>(kv_cache), M);
    return hipGetLastError();
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

}  // namespace qkvf
