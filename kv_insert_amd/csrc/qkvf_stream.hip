// A plain streaming read, for context beside the front's roofline: how fast
// this device streams a buffer with the front's launch shape (256 blocks of
// 512 threads, one per CU) and load shape (non-temporal 16-byte loads, each
// wave instruction reading 1 KB), with 16 loads per lane in flight (measured
// faster than 8: about 1.5% on 151 MB, 8% on 19 MB).  Each thread
// folds what it reads with XOR into one word of `sink`, so every byte is
// really loaded and the result can be checked on the host.
#include <hip/hip_runtime.h>

#include "qkvf_internal.h"

namespace qkvf {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kStreamThreads, 1)
stream_read(const u32x4 *__restrict__ src, int per_thread, unsigned *__restrict__ sink)
{
    // Block b reads its contiguous share; thread t its pieces t, t + 512, ...
    const u32x4 *p = src + size_t(blockIdx.x) * per_thread * kStreamThreads + threadIdx.x;
    auto at = [&](int k) { return p + size_t(k) * kStreamThreads; };
    u32x4 ring[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (j < per_thread)
            ring[j] = __builtin_nontemporal_load(at(j));
    unsigned acc = 0;
    int k = 0;
    for (; k + 16 <= per_thread; k += 16) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            acc ^= ring[j].x ^ ring[j].y ^ ring[j].z ^ ring[j].w;
            if (k + j + 16 < per_thread)
                ring[j] = __builtin_nontemporal_load(at(k + j + 16));
        }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (k + j < per_thread)
            acc ^= ring[j].x ^ ring[j].y ^ ring[j].z ^ ring[j].w;
    sink[blockIdx.x * kStreamThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, size_t bytes, unsigned *sink, hipStream_t stream)
{
    const int per_thread = int(bytes / kStreamQuantum);
    hipLaunchKernelGGL(stream_read, dim3(kGrid), dim3(kStreamThreads), 0, stream,
                       static_cast<const u32x4 *>(src), per_thread, sink);
    return hipGetLastError();
}

}  // namespace qkvf
