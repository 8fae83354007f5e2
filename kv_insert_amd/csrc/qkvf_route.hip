// gfx950 kernel of MuseRouting (cute_ops page, MuseRouting entry and class;
// unsupported_router for the constants): the routing of b <= 8 tokens over
// 256 experts.
//     score[e] = sigmoid(logit[e])          fp32: the exact sigmoid rounded once
//                                           (computed in double)
//     key[e]   = score[e] + bias[e]         fp32; the bias steers the selection
//     ids      = the 8 largest keys, best first; equal keys by lower expert id
//     weight   = score * route_scale / (sum of the 8 scores + 1e-15)
//                                           double, scores summed best first,
//                                           rounded once to fp32
// One wave per token; lane l holds experts 4 l .. 4 l + 3.  Each of the 8
// selection rounds takes a wave-wide max over 64-bit values that order by
// key and then by lower id, so the ranking needs no data-dependent branch;
// the maximum moves between lanes by DPP, not through the LDS crossbar.
#include <hip/hip_runtime.h>

#include "qkvf_internal.h"

namespace qkvf {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// An unsigned image of a float that orders as the float does (finite values;
// -0 is folded into +0 first, as the float comparison treats them equal).
__device__ inline uint32_t ordered(float f)
{
    const uint32_t b = __float_as_uint(f + 0.f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One step of a wave-wide 64-bit max: combine v with the value the DPP
// pattern CTRL brings from another lane (rows outside ROW_MASK keep v).
template <int CTRL, int ROW_MASK>
__device__ inline uint64_t max_dpp(uint64_t v)
{
    const int lo = __builtin_amdgcn_update_dpp(int(uint32_t(v)), int(uint32_t(v)), CTRL, ROW_MASK,
                                               0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(int(uint32_t(v >> 32)), int(uint32_t(v >> 32)),
                                               CTRL, ROW_MASK, 0xf, false);
    const uint64_t o = (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
    return o > v ? o : v;
}

// The wave-wide maximum, in every lane: lane swaps within quads, mirrors
// within 8 and 16 lanes, then row broadcasts carry the maximum to lane 63.
__device__ inline uint64_t wave_max_u64(uint64_t v)
{
    v = max_dpp<0xb1, 0xf>(v);    // quad_perm [1, 0, 3, 2]
    v = max_dpp<0x4e, 0xf>(v);    // quad_perm [2, 3, 0, 1]
    v = max_dpp<0x141, 0xf>(v);   // row_half_mirror
    v = max_dpp<0x140, 0xf>(v);   // row_mirror: every lane holds its row's max
    v = max_dpp<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v = max_dpp<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3: lane 63 holds the max
    const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(v)), 63);
    const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(v >> 32)), 63);
    return (uint64_t(hi) << 32) | lo;
}

__global__ void __launch_bounds__(64)
route(const float *__restrict__ logits, int64_t row_stride, const float *__restrict__ bias,
      double route_scale, int32_t *__restrict__ ids, float *__restrict__ weights)
{
    const int t = blockIdx.x, lane = threadIdx.x;
    const f32x4 lg = *reinterpret_cast<const f32x4 *>(logits + int64_t(t) * row_stride + 4 * lane);
    const f32x4 bs = *reinterpret_cast<const f32x4 *>(bias + 4 * lane);
    float score[4];
    uint64_t cand[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        score[i] = float(1.0 / (1.0 + exp(-double(lg[i]))));
        const float key = score[i] + bs[i];
        const int e = 4 * lane + i;
        cand[i] = (uint64_t(ordered(key)) << 32) | uint32_t(kRouteExperts - 1 - e);
    }
    int pick[kRouteTopK];
    float chosen[kRouteTopK];
#pragma unroll
    for (int k = 0; k < kRouteTopK; ++k) {
        uint64_t m = cand[0];
#pragma unroll
        for (int i = 1; i < 4; ++i)
            m = cand[i] > m ? cand[i] : m;
        m = wave_max_u64(m);
        const int e = kRouteExperts - 1 - int(uint32_t(m));
        // The owner's candidate drops out of later rounds: 0 is below every
        // candidate of a finite key, whose upper word is never 0, and at
        // least 248 untaken candidates remain.
        if ((e >> 2) == lane)
            cand[e & 3] = 0;
        const float mine = score[e & 3];
        chosen[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), e >> 2));
        pick[k] = e;
    }
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < kRouteTopK; ++k)
        sum += double(chosen[k]);
    if (lane < kRouteTopK) {
        int id = pick[0];
        float s = chosen[0];
#pragma unroll
        for (int k = 1; k < kRouteTopK; ++k)
            if (lane == k) {
                id = pick[k];
                s = chosen[k];
            }
        ids[t * kRouteTopK + lane] = id;
        weights[t * kRouteTopK + lane] = float(double(s) * route_scale / (sum + kRouteDivisionEps));
    }
}

}  // namespace

hipError_t launch_route(const float *logits, int64_t row_stride, const float *bias,
                        double route_scale, int tokens, int32_t *ids, float *weights,
                        hipStream_t stream)
{
    hipLaunchKernelGGL(route, dim3(tokens), dim3(64), 0, stream, logits, row_stride, bias,
                       route_scale, ids, weights);
    return hipGetLastError();
}

}  // namespace qkvf
