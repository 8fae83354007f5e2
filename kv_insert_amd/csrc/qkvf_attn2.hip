// gfx950 kernels of attn2: paged decode attention of the 8-token verify step
// fused with the weightless RMS norm of its output and the sigmoid gate
// (cute_ops page, attn2 entry: head_dim 64, 8 query heads per KV head, bf16
// cache [pages][nkv][16][128] with K | V per slot, 8 query rows per request,
// any context length L >= 8, an optional sliding window; with long contexts
// the keys are split over several blocks and merged through a workspace).
//
// Request r has L tokens; its query row t (0..7) sits at position L - 8 + t
// and attends keys [lo, L - 8 + t], lo = 0 or, with a window W,
// max(0, L - 8 + t - W + 1).  The output row is, per query head h (KV head
// h / 8), o / sqrt(mean(o^2) + eps) * sigmoid(gate), o = softmax(scale q K^T) V.
//
// attn2_split: one block of 16 waves per (key split z, KV head j, request
// r), 4 key groups x 4 query waves.  The 64 query rows are the 8 tokens x 8
// q heads of KV head j; query wave w owns q heads 2w, 2w + 1 (16 rows, row
// c = 8 (h - 2w) + t) in every key group.  The split's page offsets are
// staged in LDS per segment of keys, so K|V loads never wait on a table
// read.  Keys then stream in steps of 128 (one chunk of 32 per key group):
// each thread loads one 16-byte piece of K and of V of one slot, with
// kDepth steps of loads in flight (a register ring), and stages them in LDS
// as K [128 keys][64] and V [128 keys][64], both with their 16-byte pieces
// XOR-swizzled by key (one 16-byte write each).
// Each key group's waves then take their 32 keys:
//   S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, A = 16 keys, B = 16 query rows;
//                 lane l holds query l % 16 and keys 4 (l / 16) + v),
//   weights 2^(scale s - m) against a reference point m that trails the
//                 running max by at most 16 log2 units (rescaled only in a
//                 rare wave-uniform branch),
//   O^T += V^T P^T (A = 16 dims x the lane group's 8 keys, read from the
//                 key-major V by the transposing LDS read ds_read_b64_tr_b16;
//                 B = the lane's 8 weights as bf16 hi + lo parts, so no lane
//                 exchange is needed and the weights keep ~16 bits); the row
//                 sums come from the same parts through an all-ones A operand.
// After the loop the 4 key groups merge in LDS.  A request with one split
// has its rows finished by that block; otherwise each block writes (max,
// sum, O) per row to the workspace and attn2_merge, one wave per output row,
// combines the request's splits in split order, then applies the norm and
// the gate.  Blocks find their (request, split) either from the grid (one
// set of splits per request) or, when the requests share the launch's split
// slots, from all requests' lengths (shared_geometry below), which the merge
// works out again for itself.
#include <hip/hip_runtime.h>

#include "qkvf_internal.h"

namespace qkvf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))   // LDS pointers of the builtins

constexpr int kChunk = 32;                     // keys of one MFMA pass (two pages)
constexpr int kGroups = 4;                     // key groups (chunks) per step
constexpr int kStep = kChunk * kGroups;        // keys per step
constexpr int kThreads = 256 * kGroups;        // 4 query waves per key group
constexpr int kDepth = 2;                      // steps of loads in flight
// Page offsets are staged per segment of keys; a split of up to 4096 keys
// (a 128K context over 32 splits) is one segment, so its ring never drains
// for a restage.
constexpr int kSegKeys = 4096 / kStep * kStep; // keys per segment: whole steps
constexpr int kSegPages = kSegKeys / kPageSlots;
// Splits are whole steps of at least kAttn2MinSplitKeys keys.
constexpr int kMinSplitChunks = (kAttn2MinSplitKeys / kChunk + kGroups - 1) / kGroups * kGroups;
static_assert(kGroups >= 1 && kGroups <= 4 && kDepth >= 2 && kDepth % 2 == 0, "launch shape");
static_assert(kThreads / 8 == kStep, "one thread per 16-byte piece of K and of V");
// Buffer descriptor word 3 for raw 32-bit data, and the cache-policy bits of
// a store written through to memory (sc1).
constexpr int kBufferConfig = 0x00020000;
constexpr int kCacheSc1 = 16;
constexpr float kLog2e = 1.4426950408889634f;
// Weights are taken relative to a reference point m that trails the true
// running max by at most this many log2 units, so every weight is <= 2^16.
constexpr float kRescaleSlack = 16.f;
constexpr uint32_t kSlackBits = uint32_t(127 + 16) << 23;   // fp32 bits of 2^16

static_assert(kAttn2MaxSplits <= 64, "the merge gives each split one lane");

__device__ inline float sigmoidf(float g) { return 1.f / (1.f + __expf(-g)); }

// LDS layout of a staged step, K and V alike: [128 keys][64 dims], 16-byte
// piece p of key k at piece p ^ (k % 8), so that the 16-byte writes, the
// 16-byte K reads and the 8-byte transposing V reads each touch every bank
// equally often.
__device__ inline int kswz(int key) { return key & 7; }

// How request length L is cut for Z splits: keys from `base` (the page of
// the earliest attended key) in chunks of 32, `per` chunks per split (whole
// steps of kGroups chunks, at least kMinSplitChunks), `nz` non-empty splits.
struct Geom {
    int lo0, base, per, nz;
};

__device__ inline Geom split_geom(int L, int window, int Z)
{
    Geom g;
    g.lo0 = window > 0 ? max(0, L - 8 - window + 1) : 0;
    g.base = g.lo0 & ~(kPageSlots - 1);
    const int chunks = (L - g.base + kChunk - 1) / kChunk;
    g.per = max((chunks + Z - 1) / Z, Z > 1 ? kMinSplitChunks : chunks);
    g.per = (g.per + kGroups - 1) / kGroups * kGroups;
    g.nz = (chunks + g.per - 1) / g.per;
    return g;
}

// Inclusive prefix sum (OP = +) or prefix max over the wave's 64 lanes of
// non-negative values: shifts by 1, 2, 4 and 8 lanes within each row of 16
// (lanes without a source add 0), then row 0's last lane into row 1 and row
// 2's into row 3, then lane 31 into rows 2 and 3.  Lane 63 ends with the
// total.
template <int CTRL, int ROWS = 0xF>
__device__ inline int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}

template <bool MAX>
__device__ inline int wave_scan_i(int v)
{
    auto op = [](int a, int b) { return MAX ? max(a, b) : a + b; };
    v = op(v, dpp_i<0x111>(v));         // row_shr:1
    v = op(v, dpp_i<0x112>(v));         // row_shr:2
    v = op(v, dpp_i<0x114>(v));         // row_shr:4
    v = op(v, dpp_i<0x118>(v));         // row_shr:8
    v = op(v, dpp_i<0x142, 0xA>(v));    // row_bcast:15 into rows 1 and 3
    v = op(v, dpp_i<0x143, 0xC>(v));    // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ inline int wave_sum_i(int v) { return __builtin_amdgcn_readlane(wave_scan_i<false>(v), 63); }
__device__ inline int wave_max_i(int v) { return __builtin_amdgcn_readlane(wave_scan_i<true>(v), 63); }

// Chunks a request attends from the page of its earliest key (>= 1).
__device__ inline int request_chunks(int L, int window)
{
    const int lo0 = window > 0 ? max(0, L - 8 - window + 1) : 0;
    return (L - (lo0 & ~(kPageSlots - 1)) + kChunk - 1) / kChunk;
}

// Geometry of a launch whose R requests share Z > R split slots per KV
// head.  The split length `per` (chunks) is the shortest whole number of
// steps, at least kMinSplitChunks and at least 1 / kAttn2MaxSplits of the
// longest request, for which the requests' splits, ceil(c / per) each, fit
// in Z.  The count of splits only falls as the length grows, and at the
// longest request's length every request takes one split (R < Z), so a
// bisection over whole steps finds it; most launches stop at the first try.
// Request r's splits are the slots [off_r, off_r + nz_r) in request order.
// Every lane returns per; lane l < R also request l's length, nz and off.
struct SharedGeom {
    int per, L, nz, off;
};

__device__ inline SharedGeom shared_geometry(const int32_t *seq_lens, int R, int max_len,
                                             int window, int Z, int lane)
{
    SharedGeom g;
    g.L = lane < R ? min(max(seq_lens[lane], 8), max_len) : 8;
    const int c = lane < R ? request_chunks(g.L, window) : 0;
    const int total = wave_sum_i(c), most = wave_max_i(c);
    auto up = [](int v) { return (v + kGroups - 1) / kGroups * kGroups; };
    int lo = up(max(max((total + Z - 1) / Z, kMinSplitChunks),
                    (most + kAttn2MaxSplits - 1) / kAttn2MaxSplits));
    g.per = lo;
    g.nz = (c + lo - 1) / lo;
    if (wave_sum_i(g.nz) > Z) {
        // Some request is longer than lo (else every request has one split,
        // R < Z): at hi = its length, R splits fit.
        int hi = up(most);
        while (hi - lo > kGroups) {
            const int mid = lo + (hi - lo) / (2 * kGroups) * kGroups;
            if (wave_sum_i((c + mid - 1) / mid) <= Z)
                hi = mid;
            else
                lo = mid;
        }
        g.per = hi;
        g.nz = (c + hi - 1) / hi;
    }
    g.off = wave_scan_i<false>(g.nz) - g.nz;
    return g;
}

// Reductions of floats over the 16 lanes of a DPP row (every lane of the
// row gets the result): swap neighbours, swap pairs, mirror the half rows,
// mirror the row.  Over the wave, the four rows' results combine in a fixed
// order.
template <int CTRL>
__device__ inline float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ inline float row_sum(float v)
{
    v += dpp_f<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x141>(v);   // row_half_mirror
    v += dpp_f<0x140>(v);   // row_mirror
    return v;
}

__device__ inline float row_max(float v)
{
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}

__device__ inline float lane_f(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ inline float wave_max(float v)
{
    v = row_max(v);
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

__device__ inline float wave_sum(float v)
{
    v = row_sum(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

template <bool SHARED>
__global__ void __launch_bounds__(kThreads)
attn2_split(const __bf16 *__restrict__ q, int64_t q_stride, const __bf16 *__restrict__ gate,
            int64_t gate_stride, const __bf16 *__restrict__ kv_cache, int nkv,
            const int32_t *__restrict__ block_table, int64_t bt_stride,
            const int32_t *__restrict__ seq_lens, int R, int max_len, int window, int Z,
            float *__restrict__ ws, __bf16 *__restrict__ out, int64_t out_stride)
{
    // Two step buffers of K [128 keys][64] and V [128 keys][64];
    // after the key loop the same bytes hold the groups' O for the merge.
    __shared__ __attribute__((aligned(16))) __bf16 stage_lds[2][2 * kStep * kHeadDim];
    __shared__ int64_t pg[kSegPages];   // element offset of each page's K|V rows
    __shared__ float2 ml_lds[kGroups][64];

    const int j = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    // This block's request r, its split z, the request's length and geometry,
    // and the index f of the block's partial among a KV head's partials.
    int r, z, L, f;
    Geom geo;
    if constexpr (!SHARED) {
        r = blockIdx.z;
        z = blockIdx.x;
        f = r * Z + z;
        // A length outside [8, max_len] breaks the caller's contract; clamping
        // it keeps the block-table reads inside the rows the caller sized.
        L = min(max(seq_lens[r], 8), max_len);
        geo = split_geom(L, window, Z);
    } else {
        // Wave 0 works the launch's geometry out from all the lengths and
        // hands this block's part to the others through LDS.
        __shared__ int plan_lds[5];
        f = blockIdx.x;
        if (tid < 64) {
            const SharedGeom sg = shared_geometry(seq_lens, R, max_len, window, Z, lane);
            const uint64_t mine =
                __builtin_amdgcn_ballot_w64(lane < R && f >= sg.off && f < sg.off + sg.nz);
            const int rr = mine != 0 ? __builtin_ctzll(mine) : -1;
            const int k = rr < 0 ? 0 : rr;
            const int zk = f - __builtin_amdgcn_readlane(sg.off, k);
            const int Lk = __builtin_amdgcn_readlane(sg.L, k);
            const int nzk = __builtin_amdgcn_readlane(sg.nz, k);
            if (lane == 0) {
                plan_lds[0] = rr;
                plan_lds[1] = zk;
                plan_lds[2] = Lk;
                plan_lds[3] = sg.per;
                plan_lds[4] = nzk;
            }
        }
        __syncthreads();
        r = plan_lds[0];
        if (r < 0)
            return;   // a slot past the last split (uniform over the block)
        z = plan_lds[1];
        L = plan_lds[2];
        geo.lo0 = window > 0 ? max(0, L - 8 - window + 1) : 0;
        geo.base = geo.lo0 & ~(kPageSlots - 1);
        geo.per = plan_lds[3];
        geo.nz = plan_lds[4];
    }
    const int grp = tid >> 8;                  // key group: keys 32 grp .. of a step
    const int wq = (tid >> 6) & 3;             // query wave within the group
    const int c = lane & 15;   // query row of the wave (B column / output column)
    const int g = lane >> 4;   // lane group: which keys / dims of a chunk
    const int hh = 2 * wq + (c >> 3);          // q head within the KV group
    const int t = c & 7;                       // token of the row
    const int head = kQPerKv * j + hh;         // q head index in the row
    const int64_t row = int64_t(r) * 8 + t;
    const int pos = L - 8 + t;
    const int lo = window > 0 ? max(0, pos - window + 1) : 0;
    const int lo_last = window > 0 ? max(0, L - window) : 0;   // lo of token 7
    const float sc = 0.125f * kLog2e;          // softmax scale, in log2 units

    if (z >= geo.nz)
        return;   // nothing to attend in this split; the merge skips it
    const int first = geo.base + z * geo.per * kChunk;
    const int end = min(L, first + geo.per * kChunk);

    // After the key loop thread tid combines query cq = tid / 16, dims
    // d0 .. d0 + 3; a request with one split finishes its rows here, so its
    // gate values are fetched now, while the keys stream.
    const int cq = tid >> 4, d0 = 4 * (tid & 15);
    const int64_t crow = int64_t(r) * 8 + (cq & 7);                       // token cq % 8
    const int64_t ccol = int64_t(kQPerKv * j + (cq >> 3)) * kHeadDim + d0; // q head cq / 8
    bf16x4 gv = {};
    if (geo.nz == 1)
        gv = *reinterpret_cast<const bf16x4 *>(gate + crow * gate_stride + ccol);

    // Q^T operand: lane (c, g) holds q[row][head][32 s + 8 g .. + 7], s = 0, 1.
    const __bf16 *qrow = q + row * q_stride + int64_t(head) * kHeadDim;
    const bf16x8 qv0 = *reinterpret_cast<const bf16x8 *>(qrow + attn2_q_piece(g, 0));
    const bf16x8 qv1 = *reinterpret_cast<const bf16x8 *>(qrow + attn2_q_piece(g, 1));

    float m = -INFINITY;   // reference point of this lane's query (log2 units)
    f32x4 o[4] = {};       // O^T[16 dt + 4 g + v][c]
    f32x4 ls = {};         // running sum of the query's weights (all 4 equal)
    // A operand of all ones: its product with P^T sums the weights per query
    // on the matrix core, from the same hi + lo parts as the products with V.
    const bf16x8 ones = {__bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f),
                         __bf16(1.f), __bf16(1.f), __bf16(1.f), __bf16(1.f)};

    // Step layout: thread tid moves slot kl = tid / 8 of the step's 128 keys,
    // 16-byte part p = tid % 8 of its K (dims 8 p ..) and of its V: K rows of
    // all 128 keys, then V rows of all 128 keys (layout above).
    const int kl = tid >> 3, part = tid & 7;
    const int k_lds = kl * kHeadDim + 8 * (part ^ kswz(kl));
    const int v_lds = kStep * kHeadDim + kl * kHeadDim + 8 * (part ^ kswz(kl));
    const int kg_lds = kChunk * grp * kHeadDim;                          // group's K rows
    const int vg_lds = kStep * kHeadDim + grp * (kHeadDim * kChunk);     // group's V rows
    // The V operand comes from ds_read_b64_tr_b16: every lane supplies the
    // address of 4 consecutive elements, and within each group of 16 lanes,
    // lane c receives element c % 4 of the 4 loaded by lanes 4 e + c / 4, as
    // its element e (e = 0..3).  Lane c of lane group g therefore addresses
    // key 4 g + c / 4 (and 16 more), dims 16 dt + 4 (c % 4) .. + 3, and gets
    // dim 16 dt + c of keys 4 g .. 4 g + 3 (and 16 more).
    const int trk = 4 * g + (c >> 2);
    const int tr_off = trk * kHeadDim + 4 * (c & 1);
    const __bf16 *kv_head = kv_cache + int64_t(j) * kPageSlots * kSlotWidth + part * 8;
    const int64_t page_elems = int64_t(nkv) * kPageSlots * kSlotWidth;

    for (int seg = first; seg < end; seg += kSegKeys) {
        const int seg_end = min(end, seg + kSegKeys);
        const int page0 = seg / kPageSlots;
        const int npg = (seg_end - 1) / kPageSlots - page0 + 1;
        const int klo = max(seg, geo.lo0), khi = seg_end;   // keys loaded
        const int nst = (seg_end - seg + kStep - 1) / kStep;
        __syncthreads();   // the previous segment is done with pg
        if (tid < npg)
            pg[tid] = block_table[int64_t(r) * bt_stride + page0 + tid] * page_elems;
        __syncthreads();

        // Loads are issued unconditionally, so that the number of loads behind
        // each ring slot is the same on every path and the wait before staging
        // a slot leaves the later slots in flight; a step past the segment
        // (never staged) reads the two pieces of the block's own q head that
        // the Q operand holds, already in cache and inside the head's 64
        // values.  A key outside [klo, khi) loads a valid key and is zeroed at
        // staging.
        auto issue = [&](int k0, bool real, bf16x8 *ring) {
            const int key = min(max(k0 + kl, klo), khi - 1);
            const __bf16 *src =
                kv_head + pg[key / kPageSlots - page0] + (key & (kPageSlots - 1)) * kSlotWidth;
            const __bf16 *src_k = real ? src : qrow + attn2_q_piece(g, 0);
            const __bf16 *src_v = real ? src + kHeadDim : qrow + attn2_q_piece(g, 1);
            ring[0] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(src_k));
            ring[1] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(src_v));
        };
        auto stage = [&](int k0, int sb, const bf16x8 *ring) {
            bf16x8 kp = ring[0], vp = ring[1];
            if (k0 < klo || k0 + kStep > khi) {   // edge step (uniform)
                const bool ok = k0 + kl >= klo && k0 + kl < khi;
                kp = ok ? kp : bf16x8{};
                vp = ok ? vp : bf16x8{};
            }
            *reinterpret_cast<bf16x8 *>(&stage_lds[sb][k_lds]) = kp;
            *reinterpret_cast<bf16x8 *>(&stage_lds[sb][v_lds]) = vp;
        };

        // The group's 32 keys of a step from buffer `buf` (a constant at every
        // call): scores, online softmax, products.
        auto compute = [&](int k0, int buf) {
            const __bf16 *Ks = &stage_lds[buf][kg_lds];
            const __bf16 *Vg = &stage_lds[buf][vg_lds];
            // S^T for 32 keys: two key tiles of 16 (A row = lane % 16).
            f32x4 s[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int key = 16 * kt + c;
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                    &Ks[key * kHeadDim + 8 * (g ^ kswz(key))]);
                const bf16x8 kb = *reinterpret_cast<const bf16x8 *>(
                    &Ks[key * kHeadDim + 8 * ((4 + g) ^ kswz(key))]);
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv0, a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qv1, a, 0, 0, 0);
                s[kt] = a;
            }
            // Lane holds raw scores of keys kc + 16 kt + 4 g + v for query c.
            // Only chunks before the last row's window start or past the first
            // row's position need the mask (uniform over the group's waves).
            const int kc = k0 + kChunk * grp;
            if (kc < lo_last || kc + kChunk > L - 7) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int kp = kc + 16 * kt + 4 * g + v;
                        s[kt][v] = kp >= lo && kp <= pos ? s[kt][v] : -INFINITY;
                    }
            }
            // Weights relative to the reference point: 2^(scale s - m).  The
            // reference moves only when a weight would exceed 2^16 (tested on
            // the weights' exponent bits) or nothing has been seen yet; then
            // (a wave-uniform branch, rare) the query's 4 lane groups are
            // reduced to its exact running max, the state is rescaled and the
            // weights are taken again.
            float e[8];
            auto weights = [&](float nm) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        e[4 * kt + v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][v], sc, nm));
            };
            weights(m == -INFINITY ? 0.f : -m);
            uint32_t eb = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                eb = max(eb, __float_as_uint(e[i]));   // weights are >= 0
            if (__builtin_amdgcn_ballot_w64(m == -INFINITY || eb > kSlackBits)) {
                float mc = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                                 fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
                mc = fmaxf(mc, __shfl_xor(mc, 16, 64));
                mc = fmaxf(mc, __shfl_xor(mc, 32, 64)) * sc;   // scale > 0 keeps the max
                const float mn = m == -INFINITY || mc > m + kRescaleSlack ? mc : m;
                const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
                ls *= alpha;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    o[dt] *= alpha;
                m = mn;
                // With nothing seen yet (m = -inf) every score here is -inf too.
                weights(m == -INFINITY ? 0.f : -m);
            }
            // Each weight goes in as bf16 hi + lo parts (two products), so the
            // weights keep about 16 bits rather than bf16's 8: hi is the weight
            // truncated to bf16 (its upper 16 bits, exact), lo = weight - hi
            // (exact in fp32) rounded to bf16.
            uint32_t hw[4];
            bf16x8 pl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t b0 = __float_as_uint(e[2 * i]), b1 = __float_as_uint(e[2 * i + 1]);
                hw[i] = (b0 >> 16) | (b1 & 0xFFFF0000u);
                pl[2 * i] = __bf16(e[2 * i] - __uint_as_float(b0 & 0xFFFF0000u));
                pl[2 * i + 1] = __bf16(e[2 * i + 1] - __uint_as_float(b1 & 0xFFFF0000u));
            }
            const bf16x8 ph = __builtin_bit_cast(bf16x8, hw);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                // V^T row 16 dt + c (A row = lane % 16): keys 4 g .. and
                // 16 + 4 g .. (4 consecutive keys stay together).  The 8-byte
                // half c % 2 of piece 2 dt + (c % 4) / 2, swizzled by key.
                const int pc = 8 * ((2 * dt + ((c & 3) >> 1)) ^ kswz(trk));
                const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (LDS_AS bf16x4 *)(&Vg[tr_off + pc]));
                const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (LDS_AS bf16x4 *)(&Vg[16 * kHeadDim + tr_off + pc]));
                const bf16x8 vv = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, ph, o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pl, o[dt], 0, 0, 0);
            }
            ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ph, ls, 0, 0, 0);
            ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pl, ls, 0, 0, 0);
        };

        bf16x8 ring[kDepth][2];
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            issue(seg + d * kStep, d < nst, ring[d]);
        // Full rounds of kDepth steps keep every ring slot in one place (no
        // early exit), then the last nst % kDepth steps.
        // Step s of the segment uses buffer s % 2 (kDepth is even, and the
        // segment's first barrier leaves both buffers free).
        static_assert(kDepth % 2 == 0, "ring slot d stages into buffer d % 2");
        const int full = nst / kDepth * kDepth;
        for (int s0 = 0; s0 < full; s0 += kDepth) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int k0 = seg + (s0 + d) * kStep;
                stage(k0, d & 1, ring[d]);
                issue(k0 + kDepth * kStep, s0 + d + kDepth < nst, ring[d]);
                __syncthreads();
                compute(k0, d & 1);
            }
        }
#pragma unroll
        for (int d = 0; d < kDepth - 1; ++d) {
            if (full + d < nst) {
                const int k0 = seg + (full + d) * kStep;
                stage(k0, d & 1, ring[d]);
                __syncthreads();
                compute(k0, d & 1);
            }
        }
    }

    // The key groups' states through LDS: group grp's O^T tile of query
    // q = 8 hh + t goes to red[grp][q][dim] (fp32, the staging bytes), its
    // (m, l) to ml_lds.
    const float l = ls[0];
    float *red = reinterpret_cast<float *>(&stage_lds[0][0]);
    // (The 16-byte column c4 of row q sits at column c4 ^ (q % 16), so that
    // the 16 rows a wave writes at once fall in distinct banks.)
    const int qi = 8 * hh + t;
    __syncthreads();   // every wave is done with the staging buffers
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4 *>(
            &red[(grp * 64 + qi) * kHeadDim + 4 * ((4 * dt + g) ^ (qi & 15))]) = o[dt];
    if (g == 0)
        ml_lds[grp][qi] = make_float2(m, l);
    __syncthreads();

    // Thread tid combines query tid / 16, dims 4 (tid % 16) .. + 3.
    float mg[kGroups], M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        mg[k] = ml_lds[k][cq].x;
        M = fmaxf(M, mg[k]);
    }
    float lt = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
        const float w = mg[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg[k] - M);
        lt += w * ml_lds[k][cq].y;
        acc += w * *reinterpret_cast<const f32x4 *>(
                       &red[(k * 64 + cq) * kHeadDim + 4 * ((d0 >> 2) ^ (cq & 15))]);
    }
    if (geo.nz == 1) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        acc *= inv;
        // The 16 threads of query cq are one DPP row.
        const float ss =
            row_sum(acc[0] * acc[0] + acc[1] * acc[1] + acc[2] * acc[2] + acc[3] * acc[3]);
        const float rr = rsqrtf(ss * (1.f / kHeadDim) + kAttn2Eps);
        bf16x4 res;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            res[v] = __bf16(acc[v] * rr * sigmoidf(float(gv[v])));
        *reinterpret_cast<bf16x4 *>(out + crow * out_stride + ccol) = res;
    } else {
        // Partial of (split f, KV head, query cq): max, sum, O[64], written
        // through to memory (sc1).  The merge runs on other XCDs and reads
        // them from memory either way; plain stores would leave them dirty
        // in this XCD's L2 for the write-back at the kernel's end, which
        // measured 0.3-0.6 us slower per call on every workload.
        const __amdgpu_buffer_rsrc_t wsr = __builtin_amdgcn_make_buffer_rsrc(
            ws + (int64_t(f) * nkv + j) * 64 * kAttn2PartialFloats, 0,
            64 * kAttn2PartialFloats * int(sizeof(float)), kBufferConfig);
        const int voff = (cq * kAttn2PartialFloats) * int(sizeof(float));
        if ((tid & 15) == 0)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(M), __float_as_uint(lt)},
                                                  wsr, voff, 0, kCacheSc1);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                  __float_as_uint(acc[3])},
            wsr, voff + (4 + d0) * int(sizeof(float)), 0, kCacheSc1);   // 16-byte aligned
    }
}

// One output row from its nz splits (nz <= ZMAX, src at split 0, zstride
// floats between splits): lane z takes split z's (max, sum), lane d sums
// dimension d over the splits in split order.  All ZMAX loads of a lane are
// issued before any is used (splits past the last one read it again and
// weigh 0), so this costs one round trip to memory.
template <int ZMAX>
__device__ inline float merge_row(const float *src, int64_t zstride, int nz, int lane)
{
    const int zl = min(lane, nz - 1);
    const float2 ml = *reinterpret_cast<const float2 *>(src + zl * zstride);
    float ov[ZMAX];
#pragma unroll
    for (int zz = 0; zz < ZMAX; ++zz)
        ov[zz] = src[min(zz, nz - 1) * zstride + 4 + lane];
    const float mz = lane < nz ? ml.x : -INFINITY;
    const float M = wave_max(mz);
    const float w = mz == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mz - M);
    const float lsum = wave_sum(w * ml.y);
    float acc = 0.f;
#pragma unroll
    for (int zz = 0; zz < ZMAX; ++zz)
        acc += lane_f(w, zz) * ov[zz];   // w = 0 past nz
    return acc * (lsum > 0.f ? 1.f / lsum : 0.f);
}

// Merge the splits of each row in split order, then the norm and the gate.
// One wave per output row (request, KV head, row 8 hh + t), which works out
// the request's splits from the lengths as the split launch did (a request
// with one split was finished there) and merges them with loads sized to
// the split count, at most ZCAP.
template <bool SHARED, int ZCAP>
__global__ void __launch_bounds__(256)
attn2_merge(const __bf16 *__restrict__ gate, int64_t gate_stride, int nkv,
            const int32_t *__restrict__ seq_lens, int R, int max_len, int window, int Z,
            const float *__restrict__ ws, __bf16 *__restrict__ out, int64_t out_stride)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int id = blockIdx.x * 4 + wave;          // < R * nkv * 64 by the grid
    const int qr = id & 63, j = (id >> 6) % nkv, r = (id >> 6) / nkv;
    const int hh = qr >> 3, t = qr & 7;
    const int64_t row = int64_t(r) * 8 + t;
    const int64_t col = int64_t(kQPerKv * j + hh) * kHeadDim + lane;
    // Fetched first: nothing before the output needs it.
    const float g = float(gate[row * gate_stride + col]);
    int off, nz;                                   // 1 <= nz <= ZCAP
    if constexpr (!SHARED) {
        nz = split_geom(min(max(seq_lens[r], 8), max_len), window, Z).nz;
        off = r * Z;
    } else {
        const SharedGeom sg = shared_geometry(seq_lens, R, max_len, window, Z, lane);
        nz = __builtin_amdgcn_readlane(sg.nz, r);
        off = __builtin_amdgcn_readlane(sg.off, r);
    }
    if (nz <= 1)
        return;   // finished by its split block
    const int64_t zstride = int64_t(nkv) * 64 * kAttn2PartialFloats;
    const float *src = ws + ((int64_t(off) * nkv + j) * 64 + qr) * kAttn2PartialFloats;
    // Loads sized to the request's split count (the same on every lane).
    float o;
    if (ZCAP <= 8 || nz <= 8)
        o = merge_row<8>(src, zstride, nz, lane);
    else if (ZCAP <= 16 || nz <= 16)
        o = merge_row<16>(src, zstride, nz, lane);
    else if (ZCAP <= 32 || nz <= 32)
        o = merge_row<(ZCAP < 32 ? ZCAP : 32)>(src, zstride, nz, lane);
    else
        o = merge_row<ZCAP>(src, zstride, nz, lane);
    const float rr = rsqrtf(wave_sum(o * o) * (1.f / kHeadDim) + kAttn2Eps);
    out[row * out_stride + col] = __bf16(o * rr * sigmoidf(g));
}

}  // namespace

hipError_t launch_attn2(const void *q, int64_t q_stride, const void *gate, int64_t gate_stride,
                        const void *kv_cache, int nkv, const int32_t *block_table,
                        int64_t bt_stride, const int32_t *seq_lens, int R, int max_len,
                        int window, const Attn2Launch &l, float *ws, void *out,
                        int64_t out_stride, hipStream_t stream)
{
    // Shared slots must exceed the request count (every request has a split
    // and the split search ends); a merge needs the workspace.
    if ((l.shared && l.slots <= R) || l.zmax > kAttn2MaxSplits || (l.zmax > 1 && ws == nullptr))
        return hipErrorInvalidValue;
    const dim3 grid(l.slots, nkv, l.shared ? 1 : R);
    auto split = l.shared ? attn2_split<true> : attn2_split<false>;
    hipLaunchKernelGGL(split, grid, dim3(kThreads), 0, stream, static_cast<const __bf16 *>(q),
                       q_stride, static_cast<const __bf16 *>(gate), gate_stride,
                       static_cast<const __bf16 *>(kv_cache), nkv, block_table, bt_stride,
                       seq_lens, R, max_len, window, l.slots, ws, static_cast<__bf16 *>(out),
                       out_stride);
    if (l.zmax > 1) {
        const dim3 mgrid(R * nkv * 64 / 4);
        auto *gp = static_cast<const __bf16 *>(gate);
        auto *op = static_cast<__bf16 *>(out);
        auto merge = l.shared ? (l.zmax <= 16   ? attn2_merge<true, 16>
                                 : l.zmax <= 32 ? attn2_merge<true, 32>
                                                : attn2_merge<true, 64>)
                              : (l.zmax <= 16   ? attn2_merge<false, 16>
                                 : l.zmax <= 32 ? attn2_merge<false, 32>
                                                : attn2_merge<false, 64>);
        hipLaunchKernelGGL(merge, mgrid, dim3(256), 0, stream, gp, gate_stride, nkv, seq_lens, R,
                           max_len, window, l.slots, ws, op, out_stride);
    }
    return hipGetLastError();
}

}  // namespace qkvf
