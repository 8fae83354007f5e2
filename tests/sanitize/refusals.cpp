// Drives every entry point of libqkvfront's C ABI through its refusal paths,
// in a host-only build of qkvf_api.cpp (device launches replaced by
// launch_stubs.cpp) made with the address and undefined-behaviour
// sanitizers.  On a machine without a GPU every call that passes its
// argument checks stops at the device check.  Prints one line per failed
// expectation and exits with the number of failures.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "qkvf.h"

namespace qkvf {
extern int g_stub_launches;
}

static int failures = 0;

static void expect(const char *what, int got, int want)
{
    if (got != want) {
        std::printf("FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

static void expect_in(const char *what, int got, int a, int b)
{
    if (got != a && got != b) {
        std::printf("FAIL %s: got %d, want %d or %d\n", what, got, a, b);
        ++failures;
    }
}

int main()
{
    // Stand-in device addresses: aligned, never dereferenced.
    char *const P = reinterpret_cast<char *>(uintptr_t(1) << 20);
    const int64_t *pi64 = reinterpret_cast<const int64_t *>(P);
    const float *pf = reinterpret_cast<const float *>(P);
    const int32_t *pi32 = reinterpret_cast<const int32_t *>(P);

    // Status texts.
    for (int s = -3; s < 20; ++s)
        if (qkvf_strerror(s) == nullptr || std::strlen(qkvf_strerror(s)) == 0)
            expect("strerror text", 0, 1);

    // Shapes and plans.
    const int nkvs[] = {-1, 0, 1, 2, 3, 4, 5, 8, 16, 1 << 30};
    for (int nkv : nkvs)
        for (int M : {-5, 0, 1, 8, 16, 17, 1 << 30}) {
            const int N = 1152 * (nkv > 0 && nkv < 64 ? nkv : 1);
            const bool shape_ok = nkv == 1 || nkv == 2 || nkv == 4 || nkv == 8;
            const bool rows_ok = M >= 1 && M <= 16;
            const int want = !shape_ok ? 2 : !rows_ok ? 3 : 1;   // 1: no device here
            expect("prepare", qkvf_prepare(N, nkv, M), want);
            // the plan takes N alone: a valid column count for some nkv
            const bool n_ok = N == 1152 || N == 2304 || N == 4608 || N == 9216;
            int g = 0, s = 0, w = 0, t = 0;
            expect("plan", qkvf_plan(N, M, &g, &s, &w, &t), !n_ok ? 2 : !rows_ok ? 3 : 0);
        }
    expect("plan nulls", qkvf_plan(9216, 8, nullptr, nullptr, nullptr, nullptr), 0);
    expect("plan N", qkvf_plan(1153, 8, nullptr, nullptr, nullptr, nullptr), 2);
    expect("workspace bytes", qkvf_workspace_bytes() > 0 ? 0 : 1, 0);

    // qkvf_run: no shape bound on this thread.
    expect("run unprepared", qkvf_run(P, P, pi64, pi64, pf, P, P, 1, nullptr), 6);

    // qkvf_run_static: shape, rows, pointers, alignment, then the device.
    expect("static shape", qkvf_run_static(1000, 1, P, P, pi64, pi64, pf, P, P, 1, nullptr), 2);
    expect("static rows", qkvf_run_static(1152, 1, P, P, pi64, pi64, pf, P, P, 17, nullptr), 3);
    expect("static null", qkvf_run_static(1152, 1, nullptr, P, pi64, pi64, pf, P, P, 1, nullptr), 5);
    expect("static align", qkvf_run_static(1152, 1, P + 8, P, pi64, pi64, pf, P, P, 1, nullptr), 4);
    expect("static device", qkvf_run_static(1152, 1, P, P, pi64, pi64, pf, P, P, 1, nullptr), 1);

    // qkvf_check in its documented order.
    auto chk = [&](int N, int nkv, int M, int64_t pages, const void *x, const void *y) {
        return qkvf_check(N, nkv, M, pages, 16, x, P, pi64, pi64, pf, y, P + 4096, 0);
    };
    expect("check shape", chk(9215, 8, 8, 16, P, P), 2);
    expect("check rows", chk(9216, 8, 0, 16, P, P), 3);
    expect("check null", chk(9216, 8, 8, 16, nullptr, P), 5);
    expect("check align", chk(9216, 8, 8, 16, P + 2, P), 4);
    expect("check pages", chk(9216, 8, 8, 0, P, P), 9);
    expect("check device", chk(9216, 8, 8, 16, P, P), 1);

    // Handoff modes, spin limit, faults.
    expect("handoff 2", qkvf_set_handoff(2), 9);
    expect("handoff 0", qkvf_set_handoff(0), 0);
    expect("spin limit", qkvf_set_spin_limit(1), 0);
    expect("spin limit default", qkvf_set_spin_limit(0), 0);
    unsigned *word = reinterpret_cast<unsigned *>(P);
    expect("fault word null", qkvf_fault_word(nullptr), 5);
    expect_in("fault word", qkvf_fault_word(&word), 1, 6);
    expect("fault word cleared", word == nullptr ? 0 : 1, 0);
    expect_in("device fault", qkvf_device_fault(), 0, 1);

    // attn2.
    expect("attn2 prepare nkv", qkvf_attn2_prepare(3, 4096, 1, 0), 2);
    expect("attn2 prepare len", qkvf_attn2_prepare(8, 7, 1, 0), 2);
    expect("attn2 prepare window", qkvf_attn2_prepare(8, 4096, 1, -1), 2);
    expect("attn2 prepare reqs", qkvf_attn2_prepare(8, 4096, 65, 0), 3);
    expect("attn2 prepare device", qkvf_attn2_prepare(8, 4096, 1, 0), 1);
    expect("attn2 prepare_ex mode", qkvf_attn2_prepare_ex(8, 4096, 1, 0, 2), 9);
    expect("attn2 prepare_ex nkv", qkvf_attn2_prepare_ex(3, 4096, 1, 0, 1), 2);
    expect("attn2 prepare_ex device", qkvf_attn2_prepare_ex(8, 4096, 64, 0, 1), 1);
    expect("attn2 run unprepared",
           qkvf_attn2_run(P, 4096, P, 4096, P, pi32, 1, pi32, 1, P, 4096, nullptr), 6);
    for (int nkv : {1, 2, 4, 8})
        for (int len : {8, 9, 127, 128, 129, 2048, 4096, 32768, 131072, 1 << 30})
            for (int window : {0, 1, 7, 8, 4096, 1 << 30})
                for (int reqs : {1, 2, 3, 40, 64}) {
                    int z = -1;
                    const int st = qkvf_attn2_plan(nkv, len, window, reqs, &z);
                    if (st != 0 || z < 1 || z > 256 || (z > 1 && z <= reqs) || (reqs == 1 && z > 64))
                        expect("attn2 plan", st * 100 + z, 0);
                }
    expect("attn2 plan reqs", qkvf_attn2_plan(8, 4096, 0, 0, nullptr), 3);

    // LayerFront and routing.
    expect("lf dtype", qkvf_layer_front(P, 2, 1, nullptr, 1e-6f, reinterpret_cast<float *>(P), nullptr, P, nullptr), 2);
    expect("lf eps", qkvf_layer_front(P, 0, 1, nullptr, NAN, reinterpret_cast<float *>(P), nullptr, P, nullptr), 2);
    expect("lf rows", qkvf_layer_front(P, 0, -1, nullptr, 1e-6f, reinterpret_cast<float *>(P), nullptr, P, nullptr), 3);
    expect("lf empty", qkvf_layer_front(P, 0, 0, nullptr, 1e-6f, reinterpret_cast<float *>(P), nullptr, P, nullptr), 0);
    expect("lf null", qkvf_layer_front(nullptr, 0, 1, nullptr, 1e-6f, reinterpret_cast<float *>(P), nullptr, P, nullptr), 5);
    expect("lf align", qkvf_layer_front(P + 16, 1, 1, nullptr, 1e-6f, reinterpret_cast<float *>(P), nullptr, P, nullptr), 4);
    expect("lf device", qkvf_layer_front(P, 0, 1, nullptr, 1e-6f, reinterpret_cast<float *>(P), nullptr, P, nullptr), 1);
    int32_t *ids = reinterpret_cast<int32_t *>(P);
    float *wts = reinterpret_cast<float *>(P);
    expect("route tokens", qkvf_route(pf, 256, pf, 1.0, 0, ids, wts, nullptr), 3);
    expect("route stride", qkvf_route(pf, 255, pf, 1.0, 1, ids, wts, nullptr), 2);
    expect("route scale", qkvf_route(pf, 256, pf, INFINITY, 1, ids, wts, nullptr), 2);
    expect("route null", qkvf_route(nullptr, 256, pf, 1.0, 1, ids, wts, nullptr), 5);
    expect("route align", qkvf_route(pf, 258, pf, 1.0, 1, ids, wts, nullptr), 4);
    expect("route device", qkvf_route(pf, 256, pf, 1.0, 1, ids, wts, nullptr), 1);

    // The streaming read.
    unsigned *sink = reinterpret_cast<unsigned *>(P);
    expect("stream null", qkvf_stream_read(nullptr, 1 << 21, sink, nullptr), 5);
    expect("stream bytes", qkvf_stream_read(P, 1000, sink, nullptr), 2);
    expect("stream align", qkvf_stream_read(P + 8, size_t(1) << 21, sink, nullptr), 4);
    expect("stream device", qkvf_stream_read(P, size_t(1) << 21, sink, nullptr), 1);

    qkvf_release();
    expect("no launch reached", qkvf::g_stub_launches, 0);
    std::printf("%d failures\n", failures);
    return failures;
}
