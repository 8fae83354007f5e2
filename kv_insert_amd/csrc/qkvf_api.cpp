// C-ABI layer of libqkvfront: argument checks, per-device workspace and the
// thread's bound shape.  The checks follow the reasons the reference front
// refuses a call (qkv_front page, functions "unsupported", "hidden_rows_ok",
// "supports_shape", "kv_cache_layout_ok"; cute_ops page, supports_call and
// unsupported_projection); each becomes a status code.
#include "qkvf.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "qkvf_internal.h"

namespace {

using namespace qkvf;

constexpr int kMaxDevices = 64;

// Per-device state.  Writers hold g_mu; the launch entries read the atomic
// fields without it: a workspace is published (release) only once it is
// initialised, and a row count is marked prepared only after that.
struct DeviceState {
    std::atomic<unsigned *> ws{nullptr};
    std::atomic<bool> round_robin{false};     // blocks with equal b % 8 verified to share an XCD
    std::atomic<unsigned> prepared[9] = {};   // per nkv: bit m set once rows m are prepared
    // Split partials of attn2.  A larger workspace is published before its
    // size, so a reader that sees the size also sees a buffer of that size;
    // a replaced one is kept (a call on another thread may still use it)
    // until qkvf_release.
    std::atomic<float *> attn2_ws{nullptr};
    std::atomic<size_t> attn2_ws_floats{0};
    std::vector<float *> retired;
    int arch_ok = -1;                         // -1 unknown, 0 not gfx950, 1 gfx950
    unsigned static_ok = 0;                   // per nkv: qkvf_run_static's residency checked
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];
std::atomic<bool> g_force_coherent{false};    // qkvf_set_handoff(1)
std::atomic<unsigned> g_spin_limit{kSpinLimit};  // qkvf_set_spin_limit

// Shape bound by the last qkvf_prepare of this thread.
thread_local int t_N = 0;
thread_local int t_nkv = 0;

// attn2 configuration bound by the last qkvf_attn2_prepare of this thread.
struct Attn2Config {
    int nkv = 0, max_model_len = 0, max_reqs = 0, window = 0;
    bool invariant = false;   // split count of one request for every batch size
};
thread_local Attn2Config t_attn2;

// The device this thread last checked for qkvf_layer_front and qkvf_route
// (-1: none).
thread_local int t_lf_dev = -1;

bool valid_nkv(int nkv) { return nkv == 1 || nkv == 2 || nkv == 4 || nkv == 8; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int shape_status(int N, int nkv, int M)
{
    if (!valid_nkv(nkv) || N != cols_for(nkv))
        return QKVF_ERR_SHAPE;
    if (M < 1 || M > kMaxRows)
        return QKVF_ERR_ROWS;
    return QKVF_OK;
}

// Current device index, with its gfx950 check cached.  The caller holds g_mu.
int current_device(int *dev_out)
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0)
        return QKVF_ERR_DEVICE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QKVF_ERR_DEVICE;
    DeviceState &st = g_dev[dev];
    if (st.arch_ok < 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return QKVF_ERR_DEVICE;
        st.arch_ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    }
    if (!st.arch_ok)
        return QKVF_ERR_DEVICE;
    *dev_out = dev;
    return QKVF_OK;
}

int pointer_on_device(const void *p, int dev)
{
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of an unknown pointer
        return QKVF_ERR_MEMORY;
    }
    const bool device_mem = attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
    if (!device_mem || attr.device != dev)
        return QKVF_ERR_MEMORY;
    return QKVF_OK;
}

struct Range {
    uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range_of(const void *p, size_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}

}  // namespace

extern "C" {

int qkvf_prepare(int N, int num_kv_heads, int M)
{
    const int s = shape_status(N, num_kv_heads, M);
    if (s != QKVF_OK)
        return s;
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    const int ds = current_device(&dev);
    if (ds != QKVF_OK)
        return ds;
    DeviceState &st = g_dev[dev];
    // The kernel's blocks hand partials to each other, so all of them must be
    // resident at once: one per CU on the full 256-CU device.
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        blocks_per_cu(num_kv_heads) * cus < kGrid) {
        (void)hipGetLastError();
        return QKVF_ERR_DEVICE;
    }
    if (st.ws.load(std::memory_order_relaxed) == nullptr) {
        void *p = nullptr;
        if (hipMalloc(&p, kWorkspaceWords * sizeof(unsigned)) != hipSuccess) {
            (void)hipGetLastError();
            return QKVF_ERR_ALLOC;
        }
        // Every partial word starts empty and the fault word clear.
        if (reset_workspace(static_cast<unsigned *>(p), nullptr) != hipSuccess ||
            hipDeviceSynchronize() != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFree(p);
            return QKVF_ERR_HIP;
        }
        // Where do the kernel's blocks run?  If round robin over the XCDs,
        // blocks with equal b % 8 share an XCD, and a partial read by one of
        // them may stay in that XCD's L2.
        bool rr = false;
        if (check_placement(static_cast<unsigned *>(p) + kPlacementOffset, &rr) != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFree(p);
            return QKVF_ERR_HIP;
        }
        st.round_robin.store(rr, std::memory_order_relaxed);
        st.ws.store(static_cast<unsigned *>(p), std::memory_order_release);
    }
    st.prepared[num_kv_heads].fetch_or((2u << M) - 2u, std::memory_order_release);  // rows 1..M
    t_N = N;
    t_nkv = num_kv_heads;
    return QKVF_OK;
}

int qkvf_run(const void *x, const void *W, const int64_t *positions, const int64_t *slots,
             const float *cos_sin, void *y, void *kv_cache, int M, hipStream_t stream)
{
    if (t_nkv == 0)
        return QKVF_ERR_NOT_PREPARED;
    if (M < 1 || M > kMaxRows)
        return QKVF_ERR_ROWS;
    if (!x || !W || !positions || !slots || !y || !kv_cache)
        return QKVF_ERR_NULLPTR;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(y, 16) || !aligned(kv_cache, 16) ||
        !aligned(cos_sin, 16) || !aligned(positions, 8) || !aligned(slots, 8))
        return QKVF_ERR_ALIGN;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QKVF_ERR_DEVICE;
    const DeviceState &st = g_dev[dev];
    if (!(st.prepared[t_nkv].load(std::memory_order_acquire) & (1u << M)))
        return QKVF_ERR_NOT_PREPARED;
    unsigned *ws = st.ws.load(std::memory_order_acquire);
    if (ws == nullptr)   // released meanwhile
        return QKVF_ERR_NOT_PREPARED;
    const bool coherent = g_force_coherent.load(std::memory_order_relaxed) ||
                          !st.round_robin.load(std::memory_order_relaxed);
    const hipError_t e = launch_front(t_nkv, M, x, W, positions, slots, cos_sin, y, kv_cache,
                                      ws, coherent, g_spin_limit.load(std::memory_order_relaxed),
                                      stream);
    return e == hipSuccess ? QKVF_OK : QKVF_ERR_HIP;
}

int qkvf_run_static(int N, int num_kv_heads, const void *x, const void *W,
                    const int64_t *positions, const int64_t *slots, const float *cos_sin,
                    void *y, void *kv_cache, int M, hipStream_t stream)
{
    const int s = shape_status(N, num_kv_heads, M);
    if (s != QKVF_OK)
        return s;
    if (!x || !W || !positions || !slots || !y || !kv_cache)
        return QKVF_ERR_NULLPTR;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(y, 16) || !aligned(kv_cache, 16) ||
        !aligned(cos_sin, 16) || !aligned(positions, 8) || !aligned(slots, 8))
        return QKVF_ERR_ALIGN;
    int dev = 0;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        const int ds = current_device(&dev);
        if (ds != QKVF_OK)
            return ds;
        DeviceState &st = g_dev[dev];
        if (!(st.static_ok & (1u << num_kv_heads))) {
            int cus = 0;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                    hipSuccess ||
                blocks_per_cu(num_kv_heads) * cus < kGrid) {
                (void)hipGetLastError();
                return QKVF_ERR_DEVICE;
            }
            st.static_ok |= 1u << num_kv_heads;
        }
    }
    unsigned *ws = nullptr;
    bool rr = false;
    if (static_workspace(dev, &ws, &rr) != hipSuccess) {
        (void)hipGetLastError();
        return QKVF_ERR_HIP;
    }
    const bool coherent = g_force_coherent.load(std::memory_order_relaxed) || !rr;
    const hipError_t e = launch_front(num_kv_heads, M, x, W, positions, slots, cos_sin, y,
                                      kv_cache, ws, coherent,
                                      g_spin_limit.load(std::memory_order_relaxed), stream);
    return e == hipSuccess ? QKVF_OK : QKVF_ERR_HIP;
}

int qkvf_check(int N, int num_kv_heads, int M, int64_t pages, int64_t table_rows,
               const void *x, const void *W, const int64_t *positions, const int64_t *slots,
               const float *cos_sin, const void *y, const void *kv_cache, int read_indices)
{
    int s = shape_status(N, num_kv_heads, M);
    if (s != QKVF_OK)
        return s;
    if (!x || !W || !positions || !slots || !y || !kv_cache)
        return QKVF_ERR_NULLPTR;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(y, 16) || !aligned(kv_cache, 16) ||
        !aligned(cos_sin, 16) || !aligned(positions, 8) || !aligned(slots, 8))
        return QKVF_ERR_ALIGN;
    if (pages < 1 || (cos_sin != nullptr && table_rows < 1))
        return QKVF_ERR_RANGE;
    int dev = 0;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        s = current_device(&dev);
    }
    if (s != QKVF_OK)
        return s;
    const void *ptrs[] = {x, W, positions, slots, y, kv_cache, cos_sin};
    for (const void *p : ptrs) {
        if (p == nullptr)
            continue;
        s = pointer_on_device(p, dev);
        if (s != QKVF_OK)
            return s;
    }
    const Range ry = range_of(y, size_t(M) * N * 2);
    const Range rc = range_of(kv_cache, size_t(pages) * num_kv_heads * kPageSlots * kSlotWidth * 2);
    const Range ins[] = {
        range_of(x, size_t(M) * kHidden * 2), range_of(W, size_t(N) * kHidden * 2),
        range_of(positions, size_t(M) * 8), range_of(slots, size_t(M) * 8),
        cos_sin ? range_of(cos_sin, size_t(table_rows) * kHeadDim * 4) : Range{0, 0}};
    if (overlap(ry, rc))
        return QKVF_ERR_OVERLAP;
    for (const Range &r : ins)
        if (overlap(ry, r) || overlap(rc, r))
            return QKVF_ERR_OVERLAP;
    if (read_indices) {
        std::vector<int64_t> pos(M), sl(M);
        if (hipMemcpy(pos.data(), positions, M * sizeof(int64_t), hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(sl.data(), slots, M * sizeof(int64_t), hipMemcpyDeviceToHost) != hipSuccess) {
            (void)hipGetLastError();
            return QKVF_ERR_HIP;
        }
        for (int m = 0; m < M; ++m) {
            if (cos_sin != nullptr && (pos[m] < 0 || pos[m] >= table_rows))
                return QKVF_ERR_RANGE;
            if (sl[m] >= pages * kPageSlots)
                return QKVF_ERR_RANGE;
        }
        std::vector<int64_t> used;
        for (int64_t v : sl)
            if (v >= 0)
                used.push_back(v);
        std::sort(used.begin(), used.end());
        if (std::adjacent_find(used.begin(), used.end()) != used.end())
            return QKVF_ERR_RANGE;
    }
    return QKVF_OK;
}

const char *qkvf_strerror(int status)
{
    switch (status) {
    case QKVF_OK: return "ok";
    case QKVF_ERR_DEVICE: return "no current HIP device, or it is not a gfx950 (MI355X) with 256 CUs free for one projection block each";
    case QKVF_ERR_SHAPE: return "num_kv_heads must be 1, 2, 4 or 8 and N must be 1152 * num_kv_heads";
    case QKVF_ERR_ROWS: return "M must be in [1, 16]";
    case QKVF_ERR_ALIGN: return "x, W, y, kv_cache and cos_sin must be 16-byte aligned, positions and slots 8-byte aligned";
    case QKVF_ERR_NULLPTR: return "a required pointer is NULL";
    case QKVF_ERR_NOT_PREPARED: return "qkvf_prepare has not been called for this shape and row count on this thread and device";
    case QKVF_ERR_ALLOC: return "the device workspace could not be allocated";
    case QKVF_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case QKVF_ERR_RANGE: return "a position or slot is out of range, a slot repeats, or a mode argument is not one of its values";
    case QKVF_ERR_OVERLAP: return "y or kv_cache overlaps another operand";
    case QKVF_ERR_MEMORY: return "a pointer is not device memory of the current device";
    case QKVF_ERR_TIMEOUT: return "a call on this device gave up waiting for a partial result (its blocks could not all run, or the device placed blocks on XCDs differently than at prepare); it and every call after it stored nothing until this report";
    default: return "unknown qkvf status";
    }
}

int qkvf_plan(int N, int M, int *grid, int *k_splits, int *waves_per_block, int *tiles_per_block)
{
    int nkv = 0;
    for (int c : {1, 2, 4, 8})
        if (N == cols_for(c))
            nkv = c;
    if (nkv == 0)
        return QKVF_ERR_SHAPE;
    if (M < 1 || M > kMaxRows)
        return QKVF_ERR_ROWS;
    if (grid) *grid = kGrid;
    if (k_splits) *k_splits = splits_for(nkv, M);
    if (waves_per_block) *waves_per_block = kWaves;
    if (tiles_per_block) {
        int most = 0;
        for (int x = 0; x < 8; ++x)
            most = std::max(most, tiles_for(nkv, M, x));
        *tiles_per_block = most;
    }
    return QKVF_OK;
}

size_t qkvf_workspace_bytes(void) { return kWorkspaceWords * sizeof(unsigned); }

int qkvf_set_handoff(int mode)
{
    if (mode != 0 && mode != 1)
        return QKVF_ERR_RANGE;
    g_force_coherent.store(mode == 1, std::memory_order_relaxed);
    return QKVF_OK;
}

int qkvf_set_spin_limit(unsigned rounds)
{
    g_spin_limit.store(rounds == 0 ? kSpinLimit : rounds - 1, std::memory_order_relaxed);
    return QKVF_OK;
}

int qkvf_device_fault(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QKVF_ERR_DEVICE;
    // The prepared workspace and qkvf_run_static's, each if present.
    unsigned *spaces[2] = {g_dev[dev].ws.load(std::memory_order_acquire),
                           static_workspace_if_set(dev)};
    if (spaces[0] == nullptr && spaces[1] == nullptr)
        return QKVF_OK;
    if (hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        return QKVF_ERR_HIP;
    }
    int status = QKVF_OK;
    for (unsigned *ws : spaces) {
        if (ws == nullptr)
            continue;
        unsigned word = 0;
        if (hipMemcpy(&word, ws + kFaultWord, sizeof word, hipMemcpyDeviceToHost) != hipSuccess) {
            (void)hipGetLastError();
            return QKVF_ERR_HIP;
        }
        if (word == 0)
            continue;
        // Leave the fault state: empty every partial word (a call that gave
        // up may have left some full) and clear the fault word.
        if (reset_workspace(ws, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
            (void)hipGetLastError();
            return QKVF_ERR_HIP;
        }
        status = QKVF_ERR_TIMEOUT;
    }
    return status;
}

int qkvf_fault_word(unsigned **word)
{
    if (word == nullptr)
        return QKVF_ERR_NULLPTR;
    *word = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QKVF_ERR_DEVICE;
    unsigned *ws = g_dev[dev].ws.load(std::memory_order_acquire);
    if (ws == nullptr)
        return QKVF_ERR_NOT_PREPARED;
    *word = ws + kFaultWord;
    return QKVF_OK;
}

void qkvf_release(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = -1;
    (void)hipGetDevice(&cur);
    for (int d = 0; d < kMaxDevices; ++d) {
        DeviceState &st = g_dev[d];
        for (auto &bits : st.prepared)   // first, so no launch starts on a freed workspace
            bits.store(0);
        unsigned *ws = st.ws.exchange(nullptr);
        float *aws = st.attn2_ws.exchange(nullptr);
        st.attn2_ws_floats.store(0);
        if (ws != nullptr || aws != nullptr || !st.retired.empty()) {
            (void)hipSetDevice(d);
            (void)hipDeviceSynchronize();
            if (ws != nullptr)
                (void)hipFree(ws);
            if (aws != nullptr)
                (void)hipFree(aws);
            for (float *r : st.retired)
                (void)hipFree(r);
        }
        st.retired.clear();
        st.round_robin.store(false);
        st.arch_ok = -1;
    }
    if (cur >= 0)
        (void)hipSetDevice(cur);
    t_N = 0;
    t_nkv = 0;
    t_attn2 = Attn2Config{};
}

int qkvf_attn2_prepare(int num_kv_heads, int max_model_len, int max_reqs, int window)
{
    return qkvf_attn2_prepare_ex(num_kv_heads, max_model_len, max_reqs, window, 0);
}

int qkvf_attn2_prepare_ex(int num_kv_heads, int max_model_len, int max_reqs, int window,
                          int batch_invariant)
{
    if (batch_invariant != 0 && batch_invariant != 1)
        return QKVF_ERR_RANGE;
    if (!valid_nkv(num_kv_heads) || max_model_len < 8 || window < 0)
        return QKVF_ERR_SHAPE;
    if (max_reqs < 1 || max_reqs > kAttn2MaxReqs)
        return QKVF_ERR_ROWS;
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    const int ds = current_device(&dev);
    if (ds != QKVF_OK)
        return ds;
    DeviceState &st = g_dev[dev];
    // A window that covers every position is no window.
    const int win = window >= max_model_len ? 0 : window;
    const size_t need =
        attn2_workspace_floats(num_kv_heads, max_reqs, max_model_len, win, batch_invariant == 1);
    if (need > st.attn2_ws_floats.load(std::memory_order_relaxed)) {
        void *p = nullptr;
        if (hipMalloc(&p, need * sizeof(float)) != hipSuccess) {
            (void)hipGetLastError();
            return QKVF_ERR_ALLOC;
        }
        float *old = st.attn2_ws.exchange(static_cast<float *>(p), std::memory_order_release);
        st.attn2_ws_floats.store(need, std::memory_order_release);
        if (old != nullptr)
            st.retired.push_back(old);
    }
    t_attn2 = Attn2Config{num_kv_heads, max_model_len, max_reqs, win, batch_invariant == 1};
    return QKVF_OK;
}

int qkvf_attn2_run(const void *q, int64_t q_row_stride, const void *gate, int64_t gate_row_stride,
                   const void *kv_cache, const int32_t *block_table, int64_t block_table_stride,
                   const int32_t *seq_lens, int num_reqs, void *out, int64_t out_row_stride,
                   hipStream_t stream)
{
    const Attn2Config cfg = t_attn2;
    if (cfg.nkv == 0)
        return QKVF_ERR_NOT_PREPARED;
    if (num_reqs < 1 || num_reqs > cfg.max_reqs)
        return QKVF_ERR_ROWS;
    if (!q || !gate || !kv_cache || !block_table || !seq_lens || !out)
        return QKVF_ERR_NULLPTR;
    const int64_t width = int64_t(kQPerKv) * cfg.nkv * kHeadDim;
    if (q_row_stride < width || gate_row_stride < width || out_row_stride < width ||
        block_table_stride < 1)
        return QKVF_ERR_SHAPE;
    if (!aligned(q, 16) || q_row_stride % 8 || !aligned(gate, 8) || gate_row_stride % 4 ||
        !aligned(out, 8) || out_row_stride % 4 || !aligned(kv_cache, 16) ||
        !aligned(block_table, 4) || !aligned(seq_lens, 4))
        return QKVF_ERR_ALIGN;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QKVF_ERR_DEVICE;
    const DeviceState &st = g_dev[dev];
    const Attn2Launch l =
        attn2_launch(cfg.nkv, num_reqs, cfg.max_model_len, cfg.window, cfg.invariant);
    const size_t need = attn2_call_floats(l, cfg.nkv, num_reqs);
    // Size first: a buffer published with this size or a later, larger one.
    if (need > st.attn2_ws_floats.load(std::memory_order_acquire))
        return QKVF_ERR_NOT_PREPARED;
    float *ws = st.attn2_ws.load(std::memory_order_acquire);
    const hipError_t e = launch_attn2(q, q_row_stride, gate, gate_row_stride, kv_cache, cfg.nkv,
                                      block_table, block_table_stride, seq_lens, num_reqs,
                                      cfg.max_model_len, cfg.window, l, ws, out, out_row_stride,
                                      stream);
    return e == hipSuccess ? QKVF_OK : QKVF_ERR_HIP;
}

int qkvf_attn2_plan(int num_kv_heads, int max_model_len, int window, int num_reqs, int *splits)
{
    if (!valid_nkv(num_kv_heads) || max_model_len < 8 || window < 0)
        return QKVF_ERR_SHAPE;
    if (num_reqs < 1 || num_reqs > kAttn2MaxReqs)
        return QKVF_ERR_ROWS;
    if (splits)
        *splits = attn2_splits(num_kv_heads, num_reqs, max_model_len,
                               window >= max_model_len ? 0 : window);
    return QKVF_OK;
}

}  // extern "C"

namespace {
// The current device, checked to be a gfx950 once per thread and device.
int checked_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QKVF_ERR_DEVICE;
    if (t_lf_dev != dev) {
        std::lock_guard<std::mutex> lock(g_mu);
        int checked = 0;
        const int ds = current_device(&checked);
        if (ds != QKVF_OK)
            return ds;
        t_lf_dev = dev;
    }
    return QKVF_OK;
}
}  // namespace

int qkvf_layer_front(const void *x, int x_dtype, int64_t rows, const void *weight, float eps,
                     float *stream, float *aux, void *out, hipStream_t hip_stream)
{
    if ((x_dtype != QKVF_DTYPE_BF16 && x_dtype != QKVF_DTYPE_F32) || !(eps >= 0.f) ||
        !std::isfinite(eps))
        return QKVF_ERR_SHAPE;
    if (rows < 0 || rows > kLayerFrontMaxRows)
        return QKVF_ERR_ROWS;
    if (rows == 0)
        return QKVF_OK;
    if (!x || !stream || !out)
        return QKVF_ERR_NULLPTR;
    const bool f32 = x_dtype == QKVF_DTYPE_F32;
    if (!aligned(x, f32 ? 32 : 16) || !aligned(stream, 32) || (aux && !aligned(aux, 32)) ||
        !aligned(out, 16) || (weight && !aligned(weight, 16)))
        return QKVF_ERR_ALIGN;
    const int ds = checked_device();
    if (ds != QKVF_OK)
        return ds;
    const hipError_t e =
        launch_layer_front(x, f32, rows, weight, eps, stream, aux, out, hip_stream);
    return e == hipSuccess ? QKVF_OK : QKVF_ERR_HIP;
}

int qkvf_route(const float *logits, int64_t logits_row_stride, const float *bias,
               double route_scale, int num_tokens, int32_t *ids, float *weights,
               hipStream_t stream)
{
    if (num_tokens < 1 || num_tokens > kRouteMaxTokens)
        return QKVF_ERR_ROWS;
    if (logits_row_stride < kRouteExperts || !std::isfinite(route_scale))
        return QKVF_ERR_SHAPE;
    if (!logits || !bias || !ids || !weights)
        return QKVF_ERR_NULLPTR;
    if (!aligned(logits, 16) || logits_row_stride % 4 || !aligned(bias, 16) || !aligned(ids, 4) ||
        !aligned(weights, 4))
        return QKVF_ERR_ALIGN;
    const int ds = checked_device();
    if (ds != QKVF_OK)
        return ds;
    const hipError_t e = launch_route(logits, logits_row_stride, bias, route_scale, num_tokens,
                                      ids, weights, stream);
    return e == hipSuccess ? QKVF_OK : QKVF_ERR_HIP;
}

int qkvf_stream_read(const void *src, size_t bytes, unsigned *sink, hipStream_t stream)
{
    if (!src || !sink)
        return QKVF_ERR_NULLPTR;
    if (bytes == 0 || bytes % kStreamQuantum != 0 || bytes / kStreamQuantum > kStreamMaxQuanta)
        return QKVF_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(sink, 4))
        return QKVF_ERR_ALIGN;
    const int ds = checked_device();
    if (ds != QKVF_OK)
        return ds;
    const hipError_t e = launch_stream_read(src, bytes, sink, stream);
    return e == hipSuccess ? QKVF_OK : QKVF_ERR_HIP;
}
