// Internal interface between the C-ABI layer (qkvf_api.cpp) and the gfx950
// kernels (the front in qkvf_kernels.hip, attn2 in qkvf_attn2.hip, LayerFront
// in qkvf_layer_front.hip, MuseRouting in qkvf_route.hip).  Not installed; the
// public API is include/qkvf.h.
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace qkvf {

constexpr int kHidden = 8192;       // K of the projection
constexpr int kHeadDim = 64;        // every head is 64 columns
constexpr int kQPerKv = 8;          // q heads (and gate heads) per KV head
constexpr int kPageSlots = 16;      // slots per cache page
constexpr int kSlotWidth = 128;     // K(64) | V(64) per slot
constexpr int kMaxRows = 16;        // tokens per call
constexpr int kTileRows = 16;       // W rows per MFMA tile
constexpr int kWaves = 8;           // waves per projection block
constexpr int kGrid = 256;          // projection blocks: one per CU

// Columns for nkv KV heads: [q | k | v | gate] = 2 * (8 + 1) * nkv heads.
constexpr int cols_for(int nkv) { return 2 * (kQPerKv + 1) * nkv * kHeadDim; }
// Token rows from which x is loaded ahead of the weights; below it, with 2
// KV heads, K is split 4 ways instead of 8 (the launch picks the kernel).
constexpr int kXFirstRows = 12;
constexpr bool wide_splits(int nkv, int M) { return nkv == 2 && M < kXFirstRows; }
// K split across blocks.  For nkv >= 4 each XCD owns whole heads (18 nkv / 8
// of them) and its 32 blocks take the splits of 32 / splits row groups of
// those heads' 16-row tiles.  For nkv <= 2 (18 nkv heads do not divide by 8)
// each XCD owns N / 8 rows: whole q and k heads (their norm needs the whole
// head) filled up with v and gate rows, in 32 / splits row groups; a
// block's tiles are one short tile and 16-row tiles.
constexpr int splits_for(int nkv, int M) { return nkv == 8 || wide_splits(nkv, M) ? 4 : 8; }
// Heads of XCD x: [x heads / 8, (x + 1) heads / 8), heads = 18 nkv.
constexpr int xcd_heads(int nkv, int x) { return (x + 1) * 18 * nkv / 8 - x * 18 * nkv / 8; }
// Tiles of a block on XCD x (the same on every XCD for nkv <= 2).
constexpr int tiles_for(int nkv, int M, int x)
{
    return nkv <= 2 ? (144 * nkv / (32 / splits_for(nkv, M)) + kTileRows - 1) / kTileRows
                    : xcd_heads(nkv, x) * 4 * splits_for(nkv, M) / (kGrid / 8);
}

// Workspace layout (32-bit words): partials [splits][M][N], one fp32 word
// each (splits * N = 36864 for every nkv, M <= 16), then a sticky fault word,
// then scratch words for the placement check.  Between calls every partial
// word holds kPartialEmpty: each call's readers empty the words they consumed.
constexpr size_t kPartialWords = size_t(32) * 1152 * kMaxRows;
constexpr size_t kFaultWord = kPartialWords;
constexpr size_t kPlacementOffset = kFaultWord + 64;  // scratch of check_placement
constexpr size_t kWorkspaceWords = kPlacementOffset + kGrid;
// An empty partial word: a NaN bit pattern.  A partial whose fp32 sum has
// exactly these bits (a NaN from NaN inputs) is stored as kPartialNan.
constexpr unsigned kPartialEmpty = 0xFFFFFFFFu;
constexpr unsigned kPartialNan = 0x7FC00000u;

// Iterations (each with a short sleep) a wave waits for a partial before it
// gives up and records a fault; far longer than any call takes (about a
// second).  qkvf_set_spin_limit lowers it for tests of the failure path.
constexpr unsigned kSpinLimit = 1u << 20;

// Fault word values.
constexpr unsigned kFaultTimeout = 1;    // a wait gave up

// Enqueue one front call on `stream`.  Shapes were validated by the caller;
// ws holds kWorkspaceWords words on this device, set up by reset_workspace.
// coherent: every partial is stored write-through (the safe mode when the
// blocks with equal b % 8 are not known to share an XCD).
hipError_t launch_front(int nkv, int M, const void *x, const void *W,
                        const int64_t *positions, const int64_t *slots,
                        const float *cos_sin, void *y, void *kv_cache,
                        unsigned *ws, bool coherent, unsigned spin_limit, hipStream_t stream);

// Enqueue a kernel on `stream` that empties every partial word of ws and
// clears its fault word (no hipMemset, so it may be captured).
hipError_t reset_workspace(unsigned *ws, hipStream_t stream);

// The library's static workspace on device `dev` (current): set up at the
// first call on the device (its address, emptied, placement checked; this
// synchronizes the device), then returned at once.  Allocates nothing.
hipError_t static_workspace(int dev, unsigned **ptr, bool *round_robin);
// The static workspace of `dev` if it has been set up, else nullptr.
unsigned *static_workspace_if_set(int dev);

// Launch a kGrid-block kernel on the current device, one block per CU, and
// report whether blocks were placed on XCDs round robin (block b on XCD
// (b + c) % 8 for some c).  scratch holds kGrid words.  Synchronous.
hipError_t check_placement(unsigned *scratch, bool *round_robin);

// Projection blocks of the front kernel for nkv that one CU can hold at once
// (0 on error).  The kernel needs all kGrid blocks resident together.
int blocks_per_cu(int nkv);

// The streaming-read probe: kGrid blocks of kStreamThreads threads; a buffer
// is a whole number of kStreamQuantum bytes (one 16-byte piece per thread).
constexpr int kStreamThreads = 512;
constexpr size_t kStreamQuantum = size_t(kGrid) * kStreamThreads * 16;
constexpr size_t kStreamMaxQuanta = size_t(1) << 16;   // 128 GiB
hipError_t launch_stream_read(const void *src, size_t bytes, unsigned *sink, hipStream_t stream);

// attn2: softmax scale is 1/sqrt(64) (applied in the kernel), o-norm epsilon.
constexpr float kAttn2Eps = 1e-6f;
// A split's partial of one query row: max, sum, 2 words of padding, O[64].
constexpr int kAttn2PartialFloats = 4 + kHeadDim;
constexpr int kAttn2MaxReqs = 64;
// The 8-value piece of a 64-value query head that lane group g (0..3) holds
// in half h (0, 1) of the Q operand: values 32 h + 8 g .. + 7.  A key-loop
// step past a block's keys loads these pieces instead of a K|V slot, so
// every read of q stays inside the head's row.
constexpr int attn2_q_piece(int g, int h) { return 32 * h + 8 * g; }
static_assert(attn2_q_piece(3, 1) + 8 <= kHeadDim && attn2_q_piece(0, 0) >= 0,
              "q pieces lie inside the head");

// Key splits of an attn2 launch.  A launch aims at ~kAttn2TargetBlocks
// blocks (one 16-wave block per CU): ceil(kAttn2TargetBlocks / nkv) split
// slots per KV head.  No split is shorter than kAttn2MinSplitKeys keys (each
// split writes a 17 KB partial per KV head), so a request spans at most one
// split per kAttn2MinSplitKeys keys of the span its rows attend
// (max_model_len, or window + 7), and at most kAttn2MaxSplits.
// One request takes min(slots, its span's splits).  Several requests share
// the slots: one split length for the whole launch, the shortest (in whole
// key steps) for which all requests' splits fit, so a long request gets more
// splits than a short one and the blocks finish together.  The slot count
// depends on the deployment and the batch size only, so the launch shape of
// a batch size is fixed; shorter contexts leave trailing slots empty.  A
// layer prepared with batch-invariant splits gives every request the
// one-request split count (grid: splits x KV heads x requests), so a
// request's output bits do not depend on the other requests of its batch.
constexpr int kAttn2TargetBlocks = 256;
constexpr int kAttn2MinSplitKeys = 128;
constexpr int kAttn2MaxSplits = 64;

inline int attn2_span(int max_model_len, int window)
{
    return window > 0 && window + 7 < max_model_len ? window + 7 : max_model_len;
}

// Split slots per KV head for num_reqs requests sharing them; 1 when no
// request can take more than one split (no merge pass).  With num_reqs = 1
// it is the split count of one request.
inline int attn2_splits(int nkv, int num_reqs, int max_model_len, int window)
{
    const int span = attn2_span(max_model_len, window);
    int by_len = (span + kAttn2MinSplitKeys - 1) / kAttn2MinSplitKeys;
    if (by_len > kAttn2MaxSplits)
        by_len = kAttn2MaxSplits;
    const int per_head = (kAttn2TargetBlocks + nkv - 1) / nkv;
    const int64_t most = int64_t(num_reqs) * by_len;
    const int b = most < per_head ? int(most) : per_head;
    return b > num_reqs ? b : 1;
}

// The launch shape of a call: `slots` split blocks per KV head along grid x,
// per request (shared == false: grid slots x nkv x num_reqs) or shared by the
// requests (grid slots x nkv); zmax bounds one request's split count (1: no
// merge pass).  Shared slots always exceed num_reqs.
struct Attn2Launch {
    int slots;
    bool shared;
    int zmax;
};

inline Attn2Launch attn2_launch(int nkv, int num_reqs, int max_model_len, int window,
                                bool invariant)
{
    if (invariant || num_reqs == 1) {
        const int z = attn2_splits(nkv, 1, max_model_len, window);
        return Attn2Launch{z, false, z};
    }
    const int b = attn2_splits(nkv, num_reqs, max_model_len, window);
    if (b == 1)
        return Attn2Launch{1, false, 1};
    const int zmax = b - (num_reqs - 1);
    return Attn2Launch{b, true, zmax < kAttn2MaxSplits ? zmax : kAttn2MaxSplits};
}

// Workspace floats of a call (0: no merge pass, no workspace).
inline size_t attn2_call_floats(const Attn2Launch &l, int nkv, int num_reqs)
{
    if (l.zmax <= 1)
        return 0;
    const size_t blocks = size_t(l.shared ? 1 : num_reqs) * l.slots * nkv;
    return blocks * 64 * kAttn2PartialFloats;
}

// Workspace floats for every batch size up to max_reqs.
inline size_t attn2_workspace_floats(int nkv, int max_reqs, int max_model_len, int window,
                                     bool invariant = false)
{
    size_t most = 0;
    for (int r = 1; r <= max_reqs; ++r) {
        const size_t n =
            attn2_call_floats(attn2_launch(nkv, r, max_model_len, window, invariant), nkv, r);
        if (n > most)
            most = n;
    }
    return most;
}

// Enqueue attn2 (and its merge when l.zmax > 1) on `stream`; arguments
// validated by the caller; ws holds attn2_call_floats(l, nkv, R) floats.
hipError_t launch_attn2(const void *q, int64_t q_stride, const void *gate, int64_t gate_stride,
                        const void *kv_cache, int nkv, const int32_t *block_table,
                        int64_t bt_stride, const int32_t *seq_lens, int R, int max_len,
                        int window, const Attn2Launch &l, float *ws, void *out,
                        int64_t out_stride, hipStream_t stream);

// LayerFront: rows of kHidden values, one block per row.
constexpr int64_t kLayerFrontMaxRows = int64_t(1) << 20;
hipError_t launch_layer_front(const void *x, bool x_fp32, int64_t rows, const void *weight,
                              float eps, float *stream, float *aux, void *out,
                              hipStream_t hip_stream);

// MuseRouting: top-8 of 256 experts for up to 8 tokens, one wave per token.
constexpr int kRouteExperts = 256;
constexpr int kRouteTopK = 8;
constexpr int kRouteMaxTokens = 8;
constexpr double kRouteDivisionEps = 1e-15;
hipError_t launch_route(const float *logits, int64_t row_stride, const float *bias,
                        double route_scale, int tokens, int32_t *ids, float *weights,
                        hipStream_t stream);

}  // namespace qkvf
