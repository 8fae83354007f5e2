// gfx950 kernels of the decode-batch attention front.
//
// The projection y = x W^T for M <= 16 tokens is a weight stream: every
// element of W (up to 151 MB) is read once and meets at most 16 token values,
// so the call is bound by HBM bandwidth, not by the matrix cores.  Two
// kernels run back to back on the caller's stream:
//
//  front_partials: 256 blocks (one per CU) of 8 waves.  Block b owns a
//    contiguous K range of 8192/S (S = 32/nkv splits) and 9 row tiles of 16
//    W rows; wave w owns 1/8 of the block's K range.  Each wave keeps its
//    slice of x (16 tokens, zero-padded past M) in registers for the whole
//    kernel and streams its 9 W tiles through a register ring, one
//    v_mfma_f32_16x16x32_bf16 per 32-wide K step with W as the 16-row A
//    operand and the tokens as the 16 B columns.  The 8 wave partials of a
//    tile are summed in LDS in wave order and the block's fp32 partial goes
//    to the workspace: no atomics, fixed order.
//
//  front_epilogue: one wave per (token, 2 heads).  Sums the S partials of
//    each column in split order, rounds to bf16 (round to nearest even), and
//    for q and k heads applies the weightless RMS norm (sum of squares by a
//    butterfly of lane exchanges) and the interleaved rotation; stores the
//    row of y and the token's K|V slot.
//
// Definitions followed: qkv_front page, module summary (projection, norm,
// RoPE, y store, K/V insert) and "Structure" (partials summed in a fixed
// rank order, rounded to bf16, then the epilogue); cute_ops page, split_qkv
// (column blocks) and the attn2 contract (cache layout).
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
    static constexpr int STEPS = KW / 32;          // MFMA K steps per tile
    static constexpr int GROUPS = kGrid / S;       // row groups of 9 tiles
    // W tiles in flight per wave (register ring depth).
    static constexpr int DEPTH = STEPS >= 8 ? 3 : (STEPS >= 4 ? 5 : kTilesPerBlock);
    static_assert(S * GROUPS == kGrid, "grid covers every (split, group)");
    static_assert(GROUPS * kTilesPerBlock * kTileRows == N, "groups cover N");
    static_assert(KW % 32 == 0, "whole MFMA steps per wave");
};

__device__ inline bf16x8 load16(const __bf16 *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

template <int NKV>
__global__ void __launch_bounds__(kWaves * 64, 1)
front_partials(const __bf16 *__restrict__ x, const __bf16 *__restrict__ W,
               float *__restrict__ ws, int M)
{
    using Sh = Shape<NKV>;
    constexpr int ST = Sh::STEPS, D = Sh::DEPTH, U = kTilesPerBlock;
    const int b = blockIdx.x;
    const int split = b % Sh::S;
    const int group = b / Sh::S;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;   // A row (W row in the tile) and B column (token)
    const int q = lane >> 4;   // which 8 of the 32 K values of a step
    // K index of element j of this lane's operand in step st:
    //   kbase + st * 32 + j.  A (W) and B (x) use the same mapping, so the
    // MFMA contracts matching K values.
    const int kbase = split * Sh::KB + wave * Sh::KW + q * 8;

    bf16x8 xv[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
        if (r < M)
            xv[st] = load16(x + size_t(r) * kHidden + kbase + st * 32);
        else
            xv[st] = bf16x8{};
    }

    const __bf16 *wp = W + size_t(group * U * kTileRows + r) * kHidden + kbase;
    constexpr size_t kTileStride = size_t(kTileRows) * kHidden;

    bf16x8 ring[D][ST];
#pragma unroll
    for (int u = 0; u < D; ++u)
#pragma unroll
        for (int st = 0; st < ST; ++st)
            ring[u][st] = load16(wp + u * kTileStride + st * 32);

    // Stage u: the MFMAs of tile u, then the loads of tile u + D into the
    // registers tile u has just freed.  The scheduling barriers keep this
    // order, so (D - 1) tiles of loads stay in flight behind every MFMA.
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < ST; ++st)
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[u % D][st], xv[st], a, 0, 0, 0);
        acc[u] = a;
        if (u + D < U) {
#pragma unroll
            for (int st = 0; st < ST; ++st)
                ring[u % D][st] = load16(wp + (u + D) * kTileStride + st * 32);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Lane (r, q) holds D[row = 4q + v][token = r], v = 0..3.  Sum the 8
    // waves' tiles in wave order, one tile at a time through a 2-deep LDS
    // buffer, and write the block's partial ws[split][token][n].
    __shared__ float red[2][kWaves][kTileRows][kTileRows + 1];
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float(*slab)[kTileRows][kTileRows + 1] = red[u & 1];
#pragma unroll
        for (int v = 0; v < 4; ++v)
            slab[wave][r][4 * q + v] = acc[u][v];
        __syncthreads();
        if (tid < kTileRows * M) {
            const int tok = tid >> 4, row = tid & 15;
            float sum = slab[0][tok][row];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                sum += slab[w][tok][row];
            const int n = (group * U + u) * kTileRows + row;
            ws[(size_t(split) * M + tok) * Sh::N + n] = sum;
        }
    }
}

__device__ inline unsigned pack2(__bf16 lo, __bf16 hi)
{
    return unsigned(__builtin_bit_cast(unsigned short, lo)) |
           (unsigned(__builtin_bit_cast(unsigned short, hi)) << 16);
}

template <int NKV>
__global__ void __launch_bounds__(64)
front_epilogue(const float *__restrict__ ws, const int64_t *__restrict__ positions,
               const int64_t *__restrict__ slots, const float *__restrict__ cos_sin,
               __bf16 *__restrict__ y, __bf16 *__restrict__ kv_cache, int M)
{
    using Sh = Shape<NKV>;
    constexpr int N = Sh::N, NQ = kQPerKv * NKV;
    const int t = blockIdx.y;
    const int lane = threadIdx.x;
    const int h = 2 * blockIdx.x + (lane >> 5);  // head of this half-wave
    const int i = lane & 31;                      // rotation pair of the head
    const int n = h * kHeadDim + 2 * i;

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
        if (cos_sin != nullptr) {
            const float *row = cos_sin + positions[t] * kHeadDim;
            const float c = row[i], sn = row[32 + i];
            o0 = __bf16(n0 * c - n1 * sn);
            o1 = __bf16(n1 * c + n0 * sn);
        } else {
            o0 = __bf16(n0);
            o1 = __bf16(n1);
        }
    }
    const unsigned packed = pack2(o0, o1);
    *reinterpret_cast<unsigned *>(y + size_t(t) * N + n) = packed;

    const int64_t slot = slots[t];
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
                       static_cast<const __bf16 *>(x), static_cast<const __bf16 *>(W), ws, M);
    hipLaunchKernelGGL(front_epilogue<NKV>, dim3(Sh::N / (2 * kHeadDim), M), dim3(64), 0,
                       stream, ws, positions, slots, cos_sin, static_cast<__bf16 *>(y),
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
