// Host-only stand-ins for the kernel launchers of libqkvfront, so that the
// C-ABI layer (qkvf_api.cpp) can be built without device code, under the
// address and undefined-behaviour sanitizers, and driven through its refusal
// paths (refusals.cpp).  Every stand-in counts its calls and fails: the
// refusal paths must never reach a launch.
#include "qkvf_internal.h"

namespace qkvf {

int g_stub_launches = 0;

hipError_t launch_front(int, int, const void *, const void *, const int64_t *, const int64_t *,
                        const float *, void *, void *, unsigned *, bool, unsigned, hipStream_t)
{
    ++g_stub_launches;
    return hipErrorInvalidValue;
}

hipError_t check_placement(unsigned *, bool *)
{
    ++g_stub_launches;
    return hipErrorInvalidValue;
}

int blocks_per_cu(int) { return 1; }

hipError_t launch_stream_read(const void *, size_t, unsigned *, hipStream_t)
{
    ++g_stub_launches;
    return hipErrorInvalidValue;
}

hipError_t launch_attn2(const void *, int64_t, const void *, int64_t, const void *, int,
                        const int32_t *, int64_t, const int32_t *, int, int, int,
                        const Attn2Launch &, float *, void *, int64_t, hipStream_t)
{
    ++g_stub_launches;
    return hipErrorInvalidValue;
}

hipError_t launch_layer_front(const void *, bool, int64_t, const void *, float, float *, float *,
                              void *, hipStream_t)
{
    ++g_stub_launches;
    return hipErrorInvalidValue;
}

hipError_t launch_route(const float *, int64_t, const float *, double, int, int32_t *, float *,
                        hipStream_t)
{
    ++g_stub_launches;
    return hipErrorInvalidValue;
}

}  // namespace qkvf

namespace qkvf {

hipError_t reset_workspace(unsigned *, hipStream_t)
{
    ++g_stub_launches;
    return hipErrorInvalidValue;
}

hipError_t static_workspace(int, unsigned **, bool *)
{
    ++g_stub_launches;
    return hipErrorInvalidValue;
}

unsigned *static_workspace_if_set(int) { return nullptr; }

}  // namespace qkvf
