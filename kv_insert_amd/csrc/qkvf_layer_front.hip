// gfx950 kernel of LayerFront (layer_front page, class LayerFront and its run
// method): the first decoder layer's input.  For each row of H = 8192 values
//     stream = float(x)                 (x bf16 or fp32)
//     aux    = stream                   (when an aux buffer is given)
//     out    = bf16(stream * r * w),    r = 1 / sqrt(mean(stream^2) + eps)
// with w the pre-QKV-projection norm's bf16 weight (1 when it has none).
//
// Four blocks of 1024 threads per row; in each, thread t owns the 8
// consecutive values 8 t .. 8 t + 7 (one 16-byte bf16 or 32-byte fp32
// access, as the page's operand checks require).  Every block reads the
// whole row and reduces its sum of squares in fp32 in the same fixed order
// (within the thread, across the wave by shuffles, then the 16 wave sums in
// index order through LDS), so the result depends on the data only; block
// part p then writes only the outputs of threads 256 p .. 256 p + 255, which
// splits a row's 24 to 80 KB of stores over four CUs.  The four blocks of a
// row are placed on one XCD (consecutive blocks go to the 8 XCDs in turn, so
// rows are taken in groups of 8 and a row's parts sit 8 blocks apart): the
// row then comes from HBM once into that XCD's L2, where parts on different
// XCDs would each fetch it.  With an fp32 x passed
// as its own stream (updated in place) the stream value is x itself, so a
// block's stores never change what another block of the row reads.
#include <hip/hip_runtime.h>

#include "qkvf_internal.h"

namespace qkvf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLfThreads = kHidden / 8;   // 1024
constexpr int kLfWaves = kLfThreads / 64;
constexpr int kLfParts = 4;                 // blocks per row, each storing a quarter

template <bool FP32_IN>
__global__ void __launch_bounds__(kLfThreads)
layer_front(const void *x, const __bf16 *__restrict__ weight, float eps, float *stream,
            float *__restrict__ aux, __bf16 *__restrict__ out, int64_t rows)
{
    __shared__ float wave_ss[kLfWaves];
    const int64_t id = blockIdx.x;
    const int64_t row = id / (8 * kLfParts) * 8 + id % 8;
    const int part = int(id / 8 % kLfParts);
    if (row >= rows)
        return;   // the grid covers whole groups of 8 rows
    const int64_t base = row * kHidden + 8 * threadIdx.x;
    float s[8];
    if (FP32_IN) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(x) + base);
        const f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = a[i];
            s[4 + i] = b[i];
        }
    } else {
        const bf16x8 v = *reinterpret_cast<const bf16x8 *>(static_cast<const __bf16 *>(x) + base);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            s[i] = float(v[i]);
    }
    bf16x8 wv;
    if (weight != nullptr)
        wv = *reinterpret_cast<const bf16x8 *>(weight + 8 * threadIdx.x);

    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        ss = __builtin_fmaf(s[i], s[i], ss);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1)
        ss += __shfl_xor(ss, k, 64);
    if ((threadIdx.x & 63) == 0)
        wave_ss[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kLfWaves; ++i)
        tot += wave_ss[i];
    const float r = 1.f / __builtin_sqrtf(tot * (1.f / kHidden) + eps);
    if (int(threadIdx.x) / (kLfThreads / kLfParts) != part)
        return;   // another block of the row stores these values

    f32x4 *sp = reinterpret_cast<f32x4 *>(stream + base);
    const f32x4 lo = {s[0], s[1], s[2], s[3]}, hi = {s[4], s[5], s[6], s[7]};
    sp[0] = lo;
    sp[1] = hi;
    if (aux != nullptr) {
        f32x4 *ap = reinterpret_cast<f32x4 *>(aux + base);
        ap[0] = lo;
        ap[1] = hi;
    }
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float n = s[i] * r;
        o[i] = __bf16(weight != nullptr ? n * float(wv[i]) : n);
    }
    *reinterpret_cast<bf16x8 *>(out + base) = o;
}

}  // namespace

hipError_t launch_layer_front(const void *x, bool x_fp32, int64_t rows, const void *weight,
                              float eps, float *stream, float *aux, void *out,
                              hipStream_t hip_stream)
{
    const dim3 grid(static_cast<unsigned>((rows + 7) / 8 * 8 * kLfParts));
    auto *w = static_cast<const __bf16 *>(weight);
    auto *o = static_cast<__bf16 *>(out);
    if (x_fp32)
        hipLaunchKernelGGL(layer_front<true>, grid, dim3(kLfThreads), 0, hip_stream, x, w, eps,
                           stream, aux, o, rows);
    else
        hipLaunchKernelGGL(layer_front<false>, grid, dim3(kLfThreads), 0, hip_stream, x, w, eps,
                           stream, aux, o, rows);
    return hipGetLastError();
}

}  // namespace qkvf
