// gfx950 kernel of the decode-batch attention front.
//
// The projection y = x W^T for M <= 16 tokens is a weight stream: every
// element of W (up to 151 MB) is read once and meets at most 16 token values,
// so the call is bound by HBM bandwidth, not by the matrix cores.  One kernel
// does the whole call:
//
//  Projection: 256 blocks (one per CU, all resident together) of 8 waves.
//    The rows of W (64 per head, 18 heads per KV head) are shared out over
//    the 8 XCDs: as whole heads for 4 and 8 KV heads; for 1 and 2 KV heads,
//    whose 18 or 36 heads do not divide by 8, as N / 8 rows per XCD (whole q
//    and k heads, whose norm needs the whole head, filled up with v and gate
//    rows).  The 32 blocks of an XCD split its rows into S K splits (S = 4
//    for 8 KV heads and for 2 below 12 token rows, else 8) and row groups:
//    block b owns one split of 8192/S K values (a contiguous range with 8 KV
//    heads, interleaved 1 KB pieces otherwise) and 3 to 9 row tiles of up
//    to 16 W rows, so every partial it produces is read on its own XCD.  For
//    each tile the block
//      - loads the 16 rows with non-temporal 16-byte loads straight into
//        LDS (buffer loads with the lds bit), each wave instruction reading
//        1 KB of one row (the shape HBM streams best), into a ring of 2 or 3
//        tile buffers, so the next tiles stream while one is used; the
//        16-byte chunks land XOR-swizzled by row (each lane fetches the chunk
//        its LDS position needs), so the transposed reads below hit
//        distinct banks;
//      - reads the tile back in MFMA operand layout, each wave its own 1/8 of
//        the block's K range, and issues v_mfma_f32_16x16x32_bf16 with W as
//        the 16-row A operand and the tokens (x, held in registers for the
//        whole kernel, zero past M) as the 16 B columns.
//    The 8 wave partials of each tile are summed in LDS in wave order, and
//    the block's fp32 partials go to the workspace, one 32-bit word each.
//
//  Epilogue: each (head, pair of tokens) is one item of one wave, on the XCD
//    whose blocks produced that head's partials (with 1 or 2 KV heads the v
//    and gate rows of an XCD form items of up to 64 columns instead).  The wave fetched its
//    tokens' slots and cos|sin rows while the weights streamed; it reads the
//    S partials of each of its columns until none is empty (a bounded wait,
//    normally served by the XCD's own L2), sums them in split order, marks
//    them empty again, rounds to bf16 (round to nearest even), applies to q
//    and k heads the weightless RMS norm (sum of squares by a butterfly of
//    lane exchanges) and the interleaved rotation, and stores its part of y
//    and of the token's K|V slot.
//
//  No read-modify-write atomics, no flags, no counters and no cache
//  maintenance; every hand-off stays inside one XCD's L2.  Between calls
//  every partial word holds kPartialEmpty (a NaN pattern no partial takes:
//  a partial with those bits is stored as the
//  canonical NaN), so a word that is not empty holds this call's partial:
//  each word has one producer and one reader per call, and the reader
//  empties it after use, so every call leaves the workspace as it found it.
//  Partials are stored plainly into the XCD's L2 (written through, device-
//  coherent, only if the device did not place blocks on XCDs round robin).
//  The sums run in a fixed order, so the result depends on the launch shape
//  only.
//
//  A wave that waits too long sets the workspace's fault word and stores
//  nothing; from then on every call finds the fault word set and runs no
//  reader, so it stores no y and no cache entry (the workspace may hold
//  stray partials), until the host clears the fault and empties the
//  workspace again.
//
// Definitions followed: qkv_front page, module summary (projection, norm,
// RoPE, y store, K/V insert) and "Structure" (partials summed in a fixed
// rank order by the owner, rounded to bf16, then the epilogue; the aux warp
// that fetches slots and cos|sin rows); cute_ops page, split_qkv (column
// blocks) and the attn2 contract (cache layout).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "qkvf_internal.h"

namespace qkvf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Buffer descriptor word 3 for raw 32-bit buffer access, and the cache bits
// of a device-coherent (sc1) buffer load: it is served by the XCD's L2 when
// the writer ran on the same XCD, and sees other XCDs' write-through stores.
// kCacheNt marks a load non-temporal.
constexpr int kBufferConfig = 0x00020000;
constexpr int kCacheSc1 = 16;
constexpr int kCacheNt = 2;

constexpr float kEps = 1e-6f;

// WIDE: K split 4 ways instead of 8 with the balanced rows (2 KV heads below
// kXFirstRows token rows, chosen at launch).
template <int NKV, bool WIDE = false>
struct Shape {
    static constexpr int N = cols_for(NKV);
    static constexpr int HEADS = N / kHeadDim;     // 18 per KV head
    static constexpr int S = NKV == 8 || WIDE ? 4 : 8;   // K splits across blocks
    static constexpr int KB = kHidden / S;         // K per block
    static constexpr int KW = KB / kWaves;         // K per wave
    static constexpr int STEPS = KW / 32;          // MFMA K steps per tile and wave
    static constexpr int CHUNKS = KB / 8;          // 16-byte chunks per tile row
    static constexpr int LOADS = 2 * CHUNKS / 64;  // 1 KB loads per wave per tile (2 rows)
    static constexpr int TILE_BYTES = kTileRows * KB * 2;
    // Tiles in the LDS ring: measured on one box against rings of 2, 3 and
    // 4 tiles (with whole heads: C1 6.87 / 7.03 / 7.12 us, C2 9.13 at 2 or 3
    // against 10.04 at 4, nkv = 4 at M = 1 14.35 / 14.10 / 14.36 us; with the
    // balanced rows 3 tiles at NKV = 1 and 4 at NKV = 2 were slower again);
    // 64 KB tiles allow 2.
    static constexpr int NB = NKV == 1 || NKV == 8 || WIDE ? 2 : 3;
    // NKV >= 4: XCD x owns heads [x HEADS / 8, (x + 1) HEADS / 8); its 32
    // blocks take the S splits of 32 / S row groups of those heads' tiles.
    static constexpr int MAX_HEADS = (HEADS + 7) / 8;
    // NKV <= 2 (H not a multiple of 8): balanced rows instead.  Only the q
    // and k heads (NORM_HEADS, rows [0, 576 NKV)) need whole heads on one
    // XCD, for their norm; the v and gate rows fill the rest, so every XCD
    // owns ROWS_X = N / 8 rows.  Its 32 blocks take the S splits of GROUPS
    // row groups of GROWS rows, as TPG tiles: tile 0 holds the group's
    // first LAST rows, the others 16 each.  Every block then streams the
    // same bytes.
    static constexpr bool BAL = HEADS % 8 != 0;
    static constexpr int NORM_HEADS = (kQPerKv + 1) * NKV;
    static constexpr int ROWS_X = N / 8;
    static constexpr int GROUPS = 32 / S;
    static constexpr int GROWS = ROWS_X / GROUPS;
    static constexpr int TPG = (GROWS + kTileRows - 1) / kTileRows;
    static constexpr int LAST = GROWS - kTileRows * (TPG - 1);
    static constexpr int U_MAX = BAL ? TPG : MAX_HEADS * 4 * S / 32;   // tiles per block, at most
    static_assert(KW % 32 == 0 && CHUNKS % 16 == 0, "whole MFMA steps, whole swizzle groups");
    static_assert(!BAL || (GROWS * GROUPS == ROWS_X && LAST > 0 && LAST % 2 == 0 &&
                           64 * ((NORM_HEADS + 7) / 8) <= ROWS_X),
                  "whole row pairs per wave, every XCD's norm heads fit its rows");
    static_assert(LOADS * 64 == 2 * CHUNKS, "each wave loads exactly two tile rows");
    static_assert(BAL || ((HEADS / 8) * 4 * S % 32 == 0 && MAX_HEADS * 4 * S % 32 == 0),
                  "whole tiles per block");
    static_assert(!WIDE || BAL, "4-way splits only with the balanced rows");
};

__device__ inline bf16x8 load16(const __bf16 *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

// W is read once: its loads are non-temporal, which keeps it from displacing
// reused lines.  They go through a buffer descriptor over W with 32-bit byte
// offsets, which measured faster than global loads of 64-bit addresses with
// the same policy.

// A lane's value moved by a DPP control code within its row of 16 lanes.
template <int CTRL>
__device__ inline float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The sum of v over each half-wave (lanes 0-31, 32-63), in every lane of
// it: quad swaps, then the 8-lane and 16-lane mirrors (DPP, no LDS), then
// one swizzle that exchanges the two rows of 16 (lane ^ 16).  Each step adds
// two equal-sized partial sums, so every lane of the half ends with the same
// bits.
__device__ inline float half_wave_sum(float v)
{
    v += dpp_move<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_move<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_move<0x141>(v);   // row_half_mirror
    v += dpp_move<0x140>(v);   // row_mirror
    // ds_swizzle bit mode within 32 lanes: and 0x1F, or 0, xor 0x10
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    return v;
}

__device__ inline unsigned pack2(__bf16 lo, __bf16 hi)
{
    return unsigned(__builtin_bit_cast(unsigned short, lo)) |
           (unsigned(__builtin_bit_cast(unsigned short, hi)) << 16);
}

// XFIRST: x is loaded ahead of the weight prologue; WIDE: see Shape (both
// chosen at launch).
template <int NKV, bool XFIRST, bool WIDE>
__global__ void __launch_bounds__(kWaves * 64, 1)
front_fused(const __bf16 *__restrict__ x, const __bf16 *__restrict__ W,
            const int64_t *__restrict__ positions, const int64_t *__restrict__ slots,
            const float *__restrict__ cos_sin, __bf16 *__restrict__ y,
            __bf16 *__restrict__ kv_cache, unsigned *__restrict__ ws, int M, int coherent,
            unsigned spin_limit)
{
    using Sh = Shape<NKV, WIDE>;
    constexpr int ST = Sh::STEPS, U = Sh::U_MAX, C = Sh::CHUNKS;
    constexpr int LD = Sh::LOADS, N = Sh::N, NQ = kQPerKv * NKV;
    constexpr size_t kTileStride = size_t(kTileRows) * kHidden;
    // The LDS ring, one array per buffer: the compiler then sees that a
    // load into one buffer cannot alias reads of another, and waits only for
    // the loads into the buffer it reads.
    __shared__ __attribute__((aligned(16))) unsigned char lds0[Sh::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char lds1[Sh::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char lds2[Sh::NB > 2 ? Sh::TILE_BYTES : 16];
    __shared__ __attribute__((aligned(16))) unsigned char lds3[Sh::NB > 3 ? Sh::TILE_BYTES : 16];
    auto bufp = [&](int i) -> unsigned char * {
        return i == 0 ? lds0 : i == 1 ? lds1 : i == 2 ? lds2 : lds3;
    };
    // A block barrier without a memory fence (a fence would wait for every
    // load into LDS in flight): LDS stores of this wave done, then s_barrier;
    // the empty asm statements keep the compiler from moving memory accesses
    // across it.
    auto block_barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt unconstrained
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    unsigned *parts = ws;
    const int b = blockIdx.x;
    // Blocks are dispatched to the 8 XCDs round robin: block b runs on XCD
    // (b + c) % 8 for a c that varies between launches.  So the 32 blocks
    // with b % 8 == x share one XCD; for NKV >= 4 they own heads
    // [x H / 8, (x + 1) H / 8) (H = 18 NKV: 9 and 18 heads) and take the S
    // splits of 32 / S row groups of those heads' 16-row tiles, so the
    // partials of a head never leave that XCD's L2.  For NKV <= 2 whole
    // heads would leave 2 of the 8 XCDs (NKV = 1) or 4 (NKV = 2) with a
    // third or a quarter more rows; the balanced rows below give every
    // block the same bytes, still with every partial read on its own XCD
    // (measured on one box: C1 6.78 -> 6.46 us, M = 8 at NKV = 1 7.05 ->
    // 6.74 us, C2 9.13 -> 9.02 us).
    const int xcd = b & 7;
    const int slot_in_xcd = b >> 3;
    const int split = slot_in_xcd % Sh::S;
    const int head_lo = xcd * Sh::HEADS / 8, head_hi = (xcd + 1) * Sh::HEADS / 8;
    // tiles of this block: a constant when every XCD has as many heads
    const int ub = Sh::HEADS % 8 == 0 || Sh::BAL ? Sh::U_MAX : (head_hi - head_lo) * Sh::S / 8;
    const int tile0 = head_lo * 4 + (slot_in_xcd / Sh::S) * ub;   // its first 16-row tile
    // Balanced rows (NKV <= 2): this XCD's norm heads [nh_lo, nh_lo + nh),
    // then its nn_cnt v and gate rows from nn_start; entry i of that list is
    // W row list_row(i), and row group grp is entries [GROWS grp, + GROWS).
    const int nh_lo = xcd * Sh::NORM_HEADS / 8;
    const int nh = (xcd + 1) * Sh::NORM_HEADS / 8 - nh_lo;
    const int nn_start = Sh::NORM_HEADS * kHeadDim + Sh::ROWS_X * xcd - kHeadDim * nh_lo;
    const int nn_cnt = Sh::ROWS_X - kHeadDim * nh;
    const int grp = slot_in_xcd / Sh::S;
    auto list_row = [&](int i) {
        return i < kHeadDim * nh ? kHeadDim * nh_lo + i : nn_start + i - kHeadDim * nh;
    };
    // Row offset and row count of tile t within the block's rows.
    auto tile_off = [](int t) {
        return !Sh::BAL ? kTileRows * t : t == 0 ? 0 : Sh::LAST + kTileRows * (t - 1);
    };
    auto tile_rows = [](int t) { return !Sh::BAL || t > 0 ? kTileRows : Sh::LAST; };
    // W row (= y column) of row `row` of tile t.
    auto w_row = [&](int t, int row) {
        return Sh::BAL ? list_row(Sh::GROWS * grp + tile_off(t) + row)
                       : (tile0 + t) * kTileRows + row;
    };
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;   // A row (W row in the tile) and B column (token)
    const int q = lane >> 4;   // which 8 of the 32 K values of a step
    // Global 16-byte chunk (of a W row, or of x) of the block's chunk c.
    // With 8 KV heads a split is one contiguous K range.  With 1-4 KV heads
    // the S splits take interleaved 1 KB pieces instead (split s owns pieces
    // s, s + S, ... of every row), so sibling blocks working in step read
    // whole stretches of a row together.  Measured on one box, alternating
    // two rounds: nkv = 4 at M = 16 15.25 -> 14.80 us, at M = 1 and 8
    // 0.12-0.16 us faster, nkv = 2 0.06-0.13 us and nkv = 1 up to 0.07 us;
    // at 8 KV heads C4 was 0.15 us slower and C3 unchanged.
    auto gchunk = [&](int c) {
        return NKV <= 4 ? ((c >> 6) * Sh::S + split) * 64 + (c & 63) : split * Sh::CHUNKS + c;
    };

    // This wave's epilogue item, if any: head `head` for tokens 2 tp (lanes
    // 0-31) and 2 tp + 1 (lanes 32-63), among this XCD's heads; lane pi of
    // each half owns rotation pair pi.
    // With balanced rows the items are column groups: the XCD's norm heads,
    // then its v and gate rows in runs of up to 64 columns (a run may end
    // mid-head; lanes past its end read its last pair and store nothing).
    const int tpairs = (M + 1) >> 1;
    const int item = wave * (kGrid / 8) + slot_in_xcd;
    const int ngroups = Sh::BAL ? nh + (nn_cnt + kHeadDim - 1) / kHeadDim : head_hi - head_lo;
    const bool has_item = item < ngroups * tpairs;
    const int cg = has_item ? item / tpairs : 0;
    const int head = head_lo + cg;
    const int col0 = !Sh::BAL ? head * kHeadDim
                     : cg < nh ? (nh_lo + cg) * kHeadDim
                               : nn_start + (cg - nh) * kHeadDim;
    const int ncols = !Sh::BAL || cg < nh ? kHeadDim : min(kHeadDim, nn_cnt - (cg - nh) * kHeadDim);
    const int tok = 2 * (has_item ? item % tpairs : 0) + (lane >> 5);
    const bool tok_ok = tok < M;
    const int tok_c = tok_ok ? tok : M - 1;  // keeps the idle half's loads in bounds
    const int pi = lane & 31;
    // Unconditional loads, so nothing waits on them until they are used.
    const int64_t pos_t = positions[tok_c];
    const int64_t slot_t = slots[tok_c];

    // Chunk (8 K values) of this lane's operands in MFMA step st, among the
    // block's chunks (gchunk gives its place in the row): A (W) and B (x)
    // use the same chunk, so the MFMA contracts matching K values.
    auto chunk_of = [&](int st) { return wave * 4 * ST + st * 4 + q; };

    // Token columns r >= M repeat row M-1; their MFMA outputs are never used.
    // x comes from L2 and is first needed at tile 0's MFMAs; where it goes
    // in the prologue is chosen below.
    const int xrow = r < M ? r : M - 1;
    bf16x8 xv[ST];
    auto load_x = [&]() {
#pragma unroll
        for (int st = 0; st < ST; ++st)
            xv[st] = load16(x + size_t(xrow) * kHidden + gchunk(chunk_of(st)) * 8);
    };

    // Byte offsets into W, which is at most 9216 x 8192 bf16 (151 MB).
    static_assert(size_t(N) * kHidden * 2 < (size_t(1) << 31), "W offsets fit 31 bits");
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(W), 0, int(size_t(N) * kHidden * 2), kBufferConfig);
    const int wtile = int((size_t(tile0 * kTileRows) * kHidden) * 2);
    constexpr int kTileBytes = int(kTileStride * 2);
    // Tile t goes straight into LDS ring buffer t % NB.  Load j of a wave
    // covers 64 consecutive chunks c0 .. c0 + 63 of tile row `row` (rows 2w,
    // 2w + 1), which land, swizzled, in LDS chunks row * C + c0 + (c ^ row):
    // the 64 lanes write 1 KB of LDS in lane order, so lane l fetches the
    // chunk that belongs at c0 + l, global chunk c0 + (l ^ row) (the same
    // 1 KB of W in another lane order).
    auto issue = [&](int t) {
#pragma unroll
        for (int j = 0; j < LD; ++j) {
            const int row = 2 * wave + (j * 64) / C;
            const int c0 = (j * 64) % C;
            const int loff = (row * C + c0) * 16;
            const int coff = gchunk(c0 + (lane ^ (row & 15))) * 16;
            // Balanced rows are gathered from the XCD's list; a short tile 0
            // has no rows for the later waves (wave-uniform), and being the
            // first tile it never sits behind a wait for another.
            const int voff = Sh::BAL ? (w_row(t, row) * kHidden) * 2 + coff
                                     : wtile + t * kTileBytes + row * kHidden * 2 + coff;
            if (tile_rows(t) == kTileRows || row < tile_rows(t))
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr, (__attribute__((address_space(3))) void *)(bufp(t % Sh::NB) + loff), 16,
                    voff, 0, 0, kCacheNt);
        }
    };
    // Wait until at most `later` tiles of this wave's loads are in flight
    // (s_waitcnt takes an immediate; loads and stores count in issue order,
    // so anything issued after those tiles only makes the wait longer).
    auto wait_tiles = [&](int later) {
        auto imm = [](int v) { return (v & 15) | (((v >> 4) & 3) << 14) | 0x70 | 0xF00; };
        switch (later) {
        case 0: __builtin_amdgcn_s_waitcnt(imm(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(imm(LD)); break;
        case 2: __builtin_amdgcn_s_waitcnt(imm(2 * LD < 63 ? 2 * LD : 63)); break;
        default: __builtin_amdgcn_s_waitcnt(imm(3 * LD < 63 ? 3 * LD : 63)); break;
        }
    };
    static_assert(Sh::NB <= 4 && 3 * LD <= 63, "wait counts");
    // Order of the first loads (the launch picks XFIRST for 12 or more
    // token rows).
    if constexpr (XFIRST)
        load_x();
#pragma unroll
    for (int t = 0; t < Sh::NB - 1; ++t)
        if (t < ub)
            issue(t);
    if constexpr (!XFIRST)
        load_x();

    // The token's rotation for this lane's pair and the fault word, fetched
    // while W streams.  The barriers keep these loads behind the weight
    // prologue, so waiting for them never stalls the stream; both are first
    // needed after the stream.
    // With balanced rows (NKV <= 2) the short tile 0 is loaded by some waves
    // only, so the compiler cannot count this wave's loads exactly and would
    // wait here for most of tile 0 before the position arrives; there the
    // rotation is fetched once tile 0 has landed (in the loop below).
    __builtin_amdgcn_sched_barrier(0);
    float rc = 0.f, rs = 0.f;
    auto load_rotation = [&]() {
        // An opaque copy of the position: the compiler would otherwise
        // compute the row's address (and wait for the position) early.
        int64_t pos_u;
        asm volatile("" : "=v"(pos_u) : "0"(pos_t));
        const float *cs_row = cos_sin != nullptr ? cos_sin + pos_u * kHeadDim
                                                 : reinterpret_cast<const float *>(ws);
        rc = cs_row[pi];
        rs = cs_row[32 + pi];
    };
    if constexpr (!Sh::BAL)
        load_rotation();
    const unsigned fault_v =
        __hip_atomic_load(ws + kFaultWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_sched_barrier(0);

    // The block's partial of (tile u, token t, row): the sum of the 8 waves'
    // partials slab[w][t][row] in wave order (slab: [8][16][17]).
    auto block_sum = [&](const float *slab, int t, int row) {
        float sum = slab[t * (kTileRows + 1) + row];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            sum += slab[(w * kTileRows + t) * (kTileRows + 1) + row];
        return sum;
    };
    auto store_partial = [&](float sum, int u, int t, int row) {
        unsigned bits = __float_as_uint(sum);
        bits = bits == kPartialEmpty ? kPartialNan : bits;
        const int n = w_row(u, row);
        unsigned *dst = parts + (size_t(split) * M + t) * N + n;
        // The reader of row n runs on this XCD: a plain store is enough (the
        // reader's device-coherent load is served by the shared L2).
        if (!coherent)
            *dst = bits;
        else
            __hip_atomic_store(dst, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    constexpr int SLAB = kWaves * kTileRows * (kTileRows + 1);  // floats per tile

    // Each tile is reduced inside the loop, where LDS has spare bandwidth:
    // the 8 wave partials of tile u go to red[u & 1] right after its MFMAs
    // and, one barrier later (all waves have written them), are summed and
    // stored while later tiles stream; red[u & 1] is written again only
    // after the barriers that follow the sum.  (Keeping the sums in registers
    // and storing all 9 after the stream measured slower: 25.3 against
    // 24.9 us at M = 8, 26.8 against 26.1 us at M = 16.)  Lane (r, q) holds
    // D[row = 4q + v][token = r], v = 0..3; token columns r >= M are never
    // needed.
    //
    // Per tile u: a barrier frees the buffer of tile u - 1, tile u + NB - 1
    // is sent into it, the sum of tile u - 1 is taken, and after this wave's
    // loads of tile u have landed a second barrier waits for every wave's;
    // then the sum is stored and the MFMAs read tile u from LDS.
    __shared__ float red[2][SLAB];
    const bool summer = threadIdx.x < kTileRows * M;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u >= ub)
            break;
        // Every wave is done with tile u - 1 (its buffer is free again) and
        // has written its partials of it to red[(u - 1) & 1].
        if (u > 0)
            block_barrier();
        if (u + Sh::NB - 1 < ub)
            issue(u + Sh::NB - 1);
        const bool sum_prev = u > 0 && summer && (threadIdx.x & 15) < tile_rows(u - 1);
        float prev = 0.f;
        if (sum_prev)
            prev = block_sum(red[(u - 1) & 1], threadIdx.x >> 4, threadIdx.x & 15);
        // This wave's loads of tile u have landed, then everyone's have.
        wait_tiles(min(u + Sh::NB - 1, ub - 1) - u);
        block_barrier();
        // The sum of tile u - 1 is stored after the wait: stores count with
        // loads, so a store issued before it would be waited for too (at
        // the last tile, whose wait is for everything, that exposed the
        // store's round trip once the tile itself had landed early).
        if (sum_prev)
            store_partial(prev, u - 1, threadIdx.x >> 4, threadIdx.x & 15);
        if (Sh::BAL && u == 0)
            load_rotation();
        const unsigned char *tile = bufp(u % Sh::NB);
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int c = chunk_of(st);
            const bf16x8 w = *reinterpret_cast<const bf16x8 *>(tile + (r * C + (c ^ r)) * 16);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xv[st], a, 0, 0, 0);
        }
        if (r < M) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[u & 1][(wave * kTileRows + r) * (kTileRows + 1) + 4 * q + v] = a[v];
        }
    }
    __syncthreads();
    if (summer && (threadIdx.x & 15) < tile_rows(ub - 1))
        store_partial(block_sum(red[(ub - 1) & 1], threadIdx.x >> 4, threadIdx.x & 15),
                      ub - 1, threadIdx.x >> 4, threadIdx.x & 15);

    // A device left in the fault state by an earlier call: no reader runs,
    // so no y or cache entry is stored (partials stored above are emptied
    // when the host clears the fault).
    // The word is read here through an opaque copy: a branch on the loaded
    // value itself would make the compiler wait for it (and for every load
    // issued before it) ahead of the loop.
    unsigned fault_in;
    asm volatile("" : "=v"(fault_in) : "0"(fault_v));
    if (fault_in != 0)
        return;

    if (has_item) {
        // The S partials of this lane's two columns: poll (bounded) with
        // device-coherent loads until none is empty, then sum in split order
        // and empty them for the next call.
        const bool pair_ok = 2 * pi < ncols;
        const int n = col0 + min(2 * pi, ncols - 2);
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            parts, 0, int(sizeof(unsigned) * kPartialWords), kBufferConfig);
        const int base = (tok_c * N + n) * int(sizeof(unsigned));
        const int split_bytes = M * N * int(sizeof(unsigned));
        // One 8-byte load per split reads the two columns' words; each word
        // was stored whole and is checked on its own.
        u32x2 v[Sh::S];
        bool gave_up = false;
        for (unsigned tries = 0;; ++tries) {
            // Every round must issue its loads again: keep the compiler from
            // hoisting them out of the loop.
            asm volatile("" ::: "memory");
#pragma unroll
            for (int sp = 0; sp < Sh::S; ++sp)
                v[sp] = __builtin_amdgcn_raw_buffer_load_b64(rsrc, base + sp * split_bytes, 0,
                                                             kCacheSc1);
            // All loads are in flight before any word is looked at.
            bool empty = false;
#pragma unroll
            for (int sp = 0; sp < Sh::S; ++sp)
                empty |= (v[sp].x == kPartialEmpty) | (v[sp].y == kPartialEmpty);
            if (__all(!empty))
                break;
            if (tries >= spin_limit) {
                ws[kFaultWord] = kFaultTimeout;
                gave_up = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int sp = 0; sp < Sh::S; ++sp) {
            a0 += __uint_as_float(v[sp].x);
            a1 += __uint_as_float(v[sp].y);
        }
        // Empty the words for the next call (the lanes of a token past M read
        // token M - 1's words too, and lanes past a run's end its last pair;
        // both leave them to their own lanes).  A wave that gave up leaves
        // them: the fault state stops later calls.
        asm volatile("" ::: "memory");
        if (tok_ok && pair_ok && !gave_up) {
            unsigned char *pb = reinterpret_cast<unsigned char *>(parts) + base;
#pragma unroll
            for (int sp = 0; sp < Sh::S; ++sp)
                *reinterpret_cast<u32x2 *>(pb + sp * split_bytes) = u32x2{kPartialEmpty, kPartialEmpty};
        }
        const __bf16 p0 = __bf16(a0), p1 = __bf16(a1);
        const float f0 = float(p0), f1 = float(p1);

        // Sum of squares of the head's 64 values over the 32 lanes of the
        // half-wave (every lane ends with the same total).
        const float ss = half_wave_sum(f0 * f0 + f1 * f1);

        if (cos_sin == nullptr) {  // a layer without RoPE: norm only
            rc = 1.f;
            rs = 0.f;
        }
        const int h = n / kHeadDim;   // the item's head, or one of a run's two
        __bf16 o0 = p0, o1 = p1;
        if (h < NQ + NKV) {  // q and k heads
            const float rr = rsqrtf(ss * (1.0f / kHeadDim) + kEps);
            const float n0 = f0 * rr, n1 = f1 * rr;
            o0 = __bf16(n0 * rc - n1 * rs);
            o1 = __bf16(n1 * rc + n0 * rs);
        }
        const unsigned packed = pack2(o0, o1);
        // A wave that gave up holds stale sums: it stores nothing, so the
        // cache never receives them (its y and cache entries keep their old
        // contents and the fault word says the call failed).
        const bool store = tok_ok && pair_ok && !gave_up;
        if (store)
            *reinterpret_cast<unsigned *>(y + size_t(tok) * N + n) = packed;

        if (store && slot_t >= 0 && h >= NQ && h < NQ + 2 * NKV) {
            const int64_t page = slot_t / kPageSlots, off = slot_t % kPageSlots;
            const bool is_k = h < NQ + NKV;
            const int j = is_k ? h - NQ : h - NQ - NKV;
            __bf16 *dst = kv_cache + ((page * NKV + j) * kPageSlots + off) * kSlotWidth +
                          (is_k ? 0 : kHeadDim) + n % kHeadDim;
            *reinterpret_cast<unsigned *>(dst) = packed;
        }
    }
}

// x goes ahead of the weight prologue for kXFirstRows (12) or more token
// rows, behind it otherwise.  Measured on one box: x first took C4 25.84 ->
// 25.60 us, NKV = 4 at M = 12 15.02 -> 14.87 us and, with the balanced rows,
// NKV = 2 at M = 16 9.60 -> 9.42 us, but cost C3 0.2 us and C1 0.1 us (and
// NKV = 1 at M = 4 and 8 about 0.1 us); a runtime branch choosing the order
// inside one kernel cost C3 0.5 us.  Below 12 rows NKV = 2 splits K 4 ways
// (wide_splits): 0.05-0.15 us faster at M = 1 ... 8 (fewer, larger tiles and
// half the partials), 0.25 us slower at M = 12 and 0.3 us at M = 16, where
// each block's x doubles; at NKV = 1 slower at every M.

template <int NKV>
hipError_t launch(int M, const void *x, const void *W, const int64_t *positions,
                  const int64_t *slots, const float *cos_sin, void *y, void *kv_cache,
                  unsigned *ws, bool coherent, unsigned spin_limit, hipStream_t stream)
{
    auto kernel = M >= kXFirstRows          ? front_fused<NKV, true, false>
                  : wide_splits(NKV, M) ? front_fused<NKV, false, NKV == 2>
                                        : front_fused<NKV, false, false>;
    hipLaunchKernelGGL(kernel, dim3(kGrid), dim3(kWaves * 64), 0, stream,
                       static_cast<const __bf16 *>(x), static_cast<const __bf16 *>(W),
                       positions, slots, cos_sin, static_cast<__bf16 *>(y),
                       static_cast<__bf16 *>(kv_cache), ws, M, coherent ? 1 : 0, spin_limit);
    return hipGetLastError();
}

// Empties the partial words and clears the fault word.
__global__ void __launch_bounds__(256) reset_words(unsigned *ws)
{
    const size_t stride = size_t(gridDim.x) * blockDim.x;
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < kPartialWords; i += stride)
        ws[i] = kPartialEmpty;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        ws[kFaultWord] = 0;
}

// One block per CU, like the front kernel; each records the XCD it runs on.
__global__ void __launch_bounds__(kWaves * 64) where_blocks_run(unsigned *out)
{
    __shared__ float pad[16384];  // 64 KB
    pad[threadIdx.x] = 0.f;
    __syncthreads();
    unsigned hw_xcd;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(hw_xcd));
    if (threadIdx.x == 0)
        out[blockIdx.x] = hw_xcd + (pad[1] == 0.f ? 0u : 1u);
}

template <int NKV>
int occupancy()
{
    int n = 0, nx = 0, nw = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, front_fused<NKV, false, false>,
                                                     kWaves * 64, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nx, front_fused<NKV, true, false>,
                                                     kWaves * 64, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nw, front_fused<NKV, false, NKV == 2>,
                                                     kWaves * 64, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n < nx ? (n < nw ? n : nw) : (nx < nw ? nx : nw);
}

}  // namespace

hipError_t launch_front(int nkv, int M, const void *x, const void *W,
                        const int64_t *positions, const int64_t *slots,
                        const float *cos_sin, void *y, void *kv_cache, unsigned *ws,
                        bool coherent, unsigned spin_limit, hipStream_t stream)
{
    switch (nkv) {
    case 1: return launch<1>(M, x, W, positions, slots, cos_sin, y, kv_cache, ws, coherent, spin_limit, stream);
    case 2: return launch<2>(M, x, W, positions, slots, cos_sin, y, kv_cache, ws, coherent, spin_limit, stream);
    case 4: return launch<4>(M, x, W, positions, slots, cos_sin, y, kv_cache, ws, coherent, spin_limit, stream);
    case 8: return launch<8>(M, x, W, positions, slots, cos_sin, y, kv_cache, ws, coherent, spin_limit, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t reset_workspace(unsigned *ws, hipStream_t stream)
{
    hipLaunchKernelGGL(reset_words, dim3(kGrid), dim3(256), 0, stream, ws);
    return hipGetLastError();
}

// The workspace of qkvf_run_static: one array per device, of the same
// layout as a prepared workspace (partials of any shape the front accepts,
// the fault word and the placement scratch: kWorkspaceWords words, 2.36 MB).
// Host code uses only its device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned scratch[kWorkspaceWords];

namespace {
constexpr int kStaticDevices = 64;
std::mutex g_static_mu;
std::atomic<unsigned *> g_static_ptr[kStaticDevices] = {};
std::atomic<bool> g_static_rr[kStaticDevices] = {};
}  // namespace

hipError_t static_workspace(int dev, unsigned **ptr, bool *round_robin)
{
    if (dev < 0 || dev >= kStaticDevices)
        return hipErrorInvalidDevice;
    unsigned *p = g_static_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_static_mu);
        p = g_static_ptr[dev].load(std::memory_order_acquire);
        if (p == nullptr) {
            // Once per device, with that device current: its copy of the
            // array, emptied, and where the kernel's blocks run on it.
            void *addr = nullptr;
            hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            unsigned *q = static_cast<unsigned *>(addr);
            e = reset_workspace(q, nullptr);
            if (e == hipSuccess)
                e = hipDeviceSynchronize();
            bool rr = false;
            if (e == hipSuccess)
                e = check_placement(q + kPlacementOffset, &rr);
            if (e != hipSuccess)
                return e;
            g_static_rr[dev].store(rr, std::memory_order_relaxed);
            g_static_ptr[dev].store(q, std::memory_order_release);
            p = q;
        }
    }
    *ptr = p;
    *round_robin = g_static_rr[dev].load(std::memory_order_relaxed);
    return hipSuccess;
}

unsigned *static_workspace_if_set(int dev)
{
    return dev >= 0 && dev < kStaticDevices ? g_static_ptr[dev].load(std::memory_order_acquire)
                                            : nullptr;
}

hipError_t check_placement(unsigned *scratch, bool *round_robin)
{
    hipLaunchKernelGGL(where_blocks_run, dim3(kGrid), dim3(kWaves * 64), 0, nullptr, scratch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    unsigned host[kGrid];
    e = hipMemcpy(host, scratch, sizeof host, hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return e;
    // A rotation: block b on XCD (b + c) % 8 for one c.
    const unsigned c = (host[0] + 8) % 8;
    bool ok = host[0] < 8;
    for (int b = 0; b < kGrid; ++b)
        ok = ok && host[b] == (unsigned(b) + c) % 8;
    *round_robin = ok;
    return hipSuccess;
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
