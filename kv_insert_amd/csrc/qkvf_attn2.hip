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
// attn2_split: one block of 4 waves per (key split z, KV head j, request r).
// Its 64 query rows are the 8 tokens x 8 q heads of KV head j; wave w owns
// q heads 2w, 2w + 1 (16 rows, row c = 8 (h - 2w) + t).  The split's page
// numbers are staged in LDS first, so K|V loads never wait on a table read;
// keys then stream in chunks of 32 (two pages of 16 slots) with kDepth
// chunks of loads in flight per thread (a register ring), each chunk staged
// in LDS as K [32 keys][64] (16-byte pieces XOR-swizzled by key) and
// V^T [64][32 keys] (groups of 4 keys XOR-swizzled by dimension / 8):
//   S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, A = 16 keys, B = 16 query rows;
//                 lane l holds query l % 16 and keys 4 (l / 16) + v),
//   online softmax per query (max over the lane's 8 keys, then across the 4
//                 lane groups holding the same query),
//   O^T += V^T P^T (A = 16 dims x the lane group's 8 keys, B = the lane's 8
//                 probabilities as bf16 hi + lo parts, so no lane exchange is
//                 needed and the weights keep ~16 bits).
// With one split the block finishes its rows itself; otherwise it writes
// (max, sum, O) per row to the workspace and attn2_merge, one wave per
// output row, combines the splits in split order, then applies the norm and
// the gate.
#include <hip/hip_runtime.h>

#include "qkvf_internal.h"

namespace qkvf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32;                     // keys per step (two pages)
constexpr int kDepth = 4;                      // chunks of loads in flight
constexpr int kSegPages = 128;                 // pages staged per segment
constexpr int kSegKeys = kSegPages * kPageSlots;
constexpr int kMinSplitChunks = kAttn2MinSplitKeys / kChunk;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;           // log2 units the max may lead by

static_assert(kAttn2MaxSplits <= 64, "the merge gives each split one lane");

__device__ inline float sigmoidf(float g) { return 1.f / (1.f + __expf(-g)); }

// How request length L is cut for Z splits: keys from `base` (the page of
// the earliest attended key) in chunks of 32, `per` chunks per split (at
// least kMinSplitChunks), `nz` non-empty splits.
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
    g.nz = (chunks + g.per - 1) / g.per;
    return g;
}

__device__ inline float wave_max(float v)
{
#pragma unroll
    for (int k = 1; k < 64; k <<= 1)
        v = fmaxf(v, __shfl_xor(v, k, 64));
    return v;
}

__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int k = 1; k < 64; k <<= 1)
        v += __shfl_xor(v, k, 64);
    return v;
}

__global__ void __launch_bounds__(256)
attn2_split(const __bf16 *__restrict__ q, int64_t q_stride, const __bf16 *__restrict__ gate,
            int64_t gate_stride, const __bf16 *__restrict__ kv_cache, int nkv,
            const int32_t *__restrict__ block_table, int64_t bt_stride,
            const int32_t *__restrict__ seq_lens, int max_len, int window, int Z,
            float *__restrict__ ws, __bf16 *__restrict__ out, int64_t out_stride)
{
    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][kChunk * kHeadDim];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[2][kHeadDim * kChunk];
    __shared__ int64_t pg[kSegPages];   // element offset of each page's K|V rows

    const int z = blockIdx.x, j = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = lane & 15;   // query row of the wave (B column / output column)
    const int g = lane >> 4;   // lane group: which keys / dims of a step
    const int hh = 2 * wave + (c >> 3);       // q head within the KV group
    const int t = c & 7;                       // token of the row
    const int head = kQPerKv * j + hh;         // q head index in the row
    const int64_t row = int64_t(r) * 8 + t;
    // A length outside [8, max_len] breaks the caller's contract; clamping it
    // keeps the block-table reads inside the rows the caller sized.
    const int L = min(max(seq_lens[r], 8), max_len);
    const int pos = L - 8 + t;
    const int lo = window > 0 ? max(0, pos - window + 1) : 0;
    const int lo_last = window > 0 ? max(0, L - window) : 0;   // lo of token 7
    const float sc = 0.125f * kLog2e;          // softmax scale, in log2 units

    const Geom geo = split_geom(L, window, Z);
    if (z >= geo.nz)
        return;   // nothing to attend in this split; the merge skips it
    const int first = geo.base + z * geo.per * kChunk;
    const int end = min(L, first + geo.per * kChunk);

    // Q^T operand: lane (c, g) holds q[row][head][32 s + 8 g .. + 7], s = 0, 1.
    const __bf16 *qrow = q + row * q_stride + int64_t(head) * kHeadDim;
    const bf16x8 qv0 = *reinterpret_cast<const bf16x8 *>(qrow + 8 * g);
    const bf16x8 qv1 = *reinterpret_cast<const bf16x8 *>(qrow + 32 + 8 * g);

    float m = -INFINITY;   // running max of this lane's query (log2 units)
    float l = 0.f;         // this lane's part of the running sum
    f32x4 o[4] = {};       // O^T[16 dt + 4 g + v][c]
    int buf = 0;

    // Chunk layout: thread tid moves slot kl = tid / 8 of the chunk's 32
    // keys, 16-byte part p = tid % 8 of its K (dims 8 p ..) and of its V.
    const int kl = tid >> 3, part = tid & 7;
    const int k_lds = kl * kHeadDim + 8 * (part ^ (kl & 7));   // K swizzle
    const int v_lds = 8 * part * kChunk + (kl ^ (4 * part));    // V^T swizzle
    const __bf16 *kv_head = kv_cache + int64_t(j) * kPageSlots * kSlotWidth + part * 8;
    const int64_t page_elems = int64_t(nkv) * kPageSlots * kSlotWidth;

    for (int seg = first; seg < end; seg += kSegKeys) {
        const int seg_end = min(end, seg + kSegKeys);
        const int page0 = seg / kPageSlots;
        const int npg = (seg_end - 1) / kPageSlots - page0 + 1;
        const int klo = max(seg, geo.lo0), khi = seg_end;   // keys loaded
        const int nch = (seg_end - seg + kChunk - 1) / kChunk;
        __syncthreads();   // the previous segment is done with pg
        if (tid < npg)
            pg[tid] = block_table[int64_t(r) * bt_stride + page0 + tid] * page_elems;
        __syncthreads();

        // Loads are issued unconditionally, so that the number of loads behind
        // each ring slot is the same on every path and the wait before staging
        // a slot leaves the later slots in flight; a chunk past the segment
        // (never staged) reads the block's own q row, already in cache.  A key
        // outside [klo, khi) loads a valid key and is zeroed at staging.
        auto issue = [&](int k0, bool real, bf16x8 *ring) {
            const int key = min(max(k0 + kl, klo), khi - 1);
            const __bf16 *src =
                kv_head + pg[key / kPageSlots - page0] + (key & (kPageSlots - 1)) * kSlotWidth;
            src = real ? src : qrow + 8 * g;
            ring[0] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(src));
            ring[1] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(src + kHeadDim));
        };
        auto stage = [&](int k0, int sb, const bf16x8 *ring) {
            bf16x8 kp = ring[0], vp = ring[1];
            if (k0 < klo || k0 + kChunk > khi) {   // edge chunk (uniform)
                const bool ok = k0 + kl >= klo && k0 + kl < khi;
                kp = ok ? kp : bf16x8{};
                vp = ok ? vp : bf16x8{};
            }
            *reinterpret_cast<bf16x8 *>(&Ks[sb][k_lds]) = kp;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                Vt[sb][v_lds + e * kChunk] = vp[e];
        };

        // One chunk from LDS buffer `buf`: scores, online softmax, products.
        auto compute = [&](int k0) {
            // S^T for 32 keys: two key tiles of 16 (A row = lane % 16).
            f32x4 s[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int key = 16 * kt + c;
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                    &Ks[buf][key * kHeadDim + 8 * (g ^ (key & 7))]);
                const bf16x8 kb = *reinterpret_cast<const bf16x8 *>(
                    &Ks[buf][key * kHeadDim + 8 * ((4 + g) ^ (key & 7))]);
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv0, a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qv1, a, 0, 0, 0);
                s[kt] = a;
            }
            // Lane holds raw scores of keys k0 + 16 kt + 4 g + v for query c.
            // Only chunks before the last row's window start or past the first
            // row's position need the mask (a uniform test).
            if (k0 < lo_last || k0 + kChunk > L - 7) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int kp = k0 + 16 * kt + 4 * g + v;
                        s[kt][v] = kp >= lo && kp <= pos ? s[kt][v] : -INFINITY;
                    }
            }
            // The reference point m moves only when a scaled score exceeds it
            // by more than 2^8, so the weights stay <= 256 and the state is
            // rescaled rarely.  Each lane tests its own 8 keys; only when some
            // lane of the wave needs more (a wave-uniform branch) are the
            // query's 4 lane groups reduced to the new reference.
            const float mo = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
            if (__builtin_amdgcn_ballot_w64(mo * sc > m + kRescaleSlack)) {
                float mc = fmaxf(mo, __shfl_xor(mo, 16, 64));
                mc = fmaxf(mc, __shfl_xor(mc, 32, 64)) * sc;   // scale > 0 keeps the max
                const float mn = mc > m + kRescaleSlack ? mc : m;
                const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    o[dt] *= alpha;
                m = mn;
            }
            // With nothing seen yet (m = -inf) every score here is -inf too.
            const float nm = m == -INFINITY ? 0.f : -m;
            // Each weight goes in as bf16 hi + lo parts (two products), so the
            // weights keep about 16 bits rather than bf16's 8: hi is the weight
            // truncated to bf16 (its upper 16 bits, exact), lo = weight - hi
            // (exact in fp32) rounded to bf16.
            float e[8];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    e[4 * kt + v] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][v], sc, nm));
                    l += e[4 * kt + v];
                }
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
                // 16 + 4 g .., stored at key group ^ (row / 8).
                const int d = 16 * dt + c;
                const int h = d >> 3;
                const bf16x4 va = *reinterpret_cast<const bf16x4 *>(
                    &Vt[buf][d * kChunk + 4 * (g ^ h)]);
                const bf16x4 vb = *reinterpret_cast<const bf16x4 *>(
                    &Vt[buf][d * kChunk + 4 * ((4 + g) ^ h)]);
                const bf16x8 vv = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, ph, o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pl, o[dt], 0, 0, 0);
            }
        };

        bf16x8 ring[kDepth][2];
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            issue(seg + d * kChunk, d < nch, ring[d]);
        // Full rounds of kDepth chunks keep every ring slot in one place (no
        // early exit), then the last nch % kDepth chunks.
        const int full = nch / kDepth * kDepth;
        for (int c0 = 0; c0 < full; c0 += kDepth) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int k0 = seg + (c0 + d) * kChunk;
                stage(k0, buf, ring[d]);
                issue(k0 + kDepth * kChunk, c0 + d + kDepth < nch, ring[d]);
                __syncthreads();
                compute(k0);
                buf ^= 1;   // the next chunk stages into the other buffer
            }
        }
#pragma unroll
        for (int d = 0; d < kDepth - 1; ++d) {
            if (full + d < nch) {
                const int k0 = seg + (full + d) * kChunk;
                stage(k0, buf, ring[d]);
                __syncthreads();
                compute(k0);
                buf ^= 1;
            }
        }
    }

    // Totals of the query across its 4 lane groups.
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    // Lane (c, g) holds O^T[16 dt + 4 g + v][c]: dims 16 dt + 4 g + v.
    if (Z == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float ss = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                o[dt][v] *= inv;
                ss += o[dt][v] * o[dt][v];
            }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float rr = rsqrtf(ss * (1.f / kHeadDim) + kAttn2Eps);
        const __bf16 *grow = gate + row * gate_stride + int64_t(head) * kHeadDim;
        __bf16 *orow = out + row * out_stride + int64_t(head) * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int d0 = 16 * dt + 4 * g;
            const bf16x4 gv = *reinterpret_cast<const bf16x4 *>(grow + d0);
            bf16x4 res;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                res[v] = __bf16(o[dt][v] * rr * sigmoidf(float(gv[v])));
            *reinterpret_cast<bf16x4 *>(orow + d0) = res;
        }
    } else {
        // Partial of (request, KV head, split, row 8 hh + t): max, sum, O[64].
        float *dst = ws + (((int64_t(r) * nkv + j) * Z + z) * 64 + 8 * hh + t) * kAttn2PartialFloats;
        if (g == 0) {
            dst[0] = m;
            dst[1] = l;
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            *reinterpret_cast<f32x4 *>(dst + 4 + 16 * dt + 4 * g) = o[dt];  // 16-byte aligned
    }
}

// Merge the non-empty splits of each row in split order, then the norm and
// the gate.  One wave per output row (request, KV head, row 8 hh + t): lane
// z reads split z's (max, sum), lane d accumulates dimension d.  All ZMAX
// loads of a lane are issued before any is used (splits past the last
// non-empty one read it again with weight 0), so the merge costs one round
// trip to memory.
template <int ZMAX>
__global__ void __launch_bounds__(256)
attn2_merge(const __bf16 *__restrict__ gate, int64_t gate_stride, int nkv,
            const int32_t *__restrict__ seq_lens, int max_len, int window, int Z,
            const float *__restrict__ ws, __bf16 *__restrict__ out, int64_t out_stride)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int id = blockIdx.x * 4 + wave;          // < R * nkv * 64 by the grid
    const int qr = id & 63, j = (id >> 6) % nkv, r = (id >> 6) / nkv;
    const int hh = qr >> 3, t = qr & 7;
    const int L = min(max(seq_lens[r], 8), max_len);
    const int nz = split_geom(L, window, Z).nz;   // 1 <= nz <= Z <= ZMAX
    const float *src = ws + ((int64_t(r) * nkv + j) * Z * 64 + qr) * kAttn2PartialFloats;
    const int64_t zstride = int64_t(64) * kAttn2PartialFloats;

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
        acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), zz)) * ov[zz];
    const float o = acc * (lsum > 0.f ? 1.f / lsum : 0.f);
    const float rr = rsqrtf(wave_sum(o * o) * (1.f / kHeadDim) + kAttn2Eps);
    const int64_t row = int64_t(r) * 8 + t;
    const int64_t col = int64_t(kQPerKv * j + hh) * kHeadDim + lane;
    out[row * out_stride + col] = __bf16(o * rr * sigmoidf(float(gate[row * gate_stride + col])));
}

}  // namespace

hipError_t launch_attn2(const void *q, int64_t q_stride, const void *gate, int64_t gate_stride,
                        const void *kv_cache, int nkv, const int32_t *block_table,
                        int64_t bt_stride, const int32_t *seq_lens, int R, int max_len,
                        int window, int Z, float *ws, void *out, int64_t out_stride,
                        hipStream_t stream)
{
    hipLaunchKernelGGL(attn2_split, dim3(Z, nkv, R), dim3(256), 0, stream,
                       static_cast<const __bf16 *>(q), q_stride, static_cast<const __bf16 *>(gate),
                       gate_stride, static_cast<const __bf16 *>(kv_cache), nkv, block_table,
                       bt_stride, seq_lens, max_len, window, Z, ws, static_cast<__bf16 *>(out),
                       out_stride);
    if (Z > 1) {
        const dim3 grid(R * nkv * 64 / 4);
        auto *gp = static_cast<const __bf16 *>(gate);
        auto *op = static_cast<__bf16 *>(out);
        if (Z <= 16)
            hipLaunchKernelGGL(attn2_merge<16>, grid, dim3(256), 0, stream, gp, gate_stride, nkv,
                               seq_lens, max_len, window, Z, ws, op, out_stride);
        else if (Z <= 32)
            hipLaunchKernelGGL(attn2_merge<32>, grid, dim3(256), 0, stream, gp, gate_stride, nkv,
                               seq_lens, max_len, window, Z, ws, op, out_stride);
        else
            hipLaunchKernelGGL(attn2_merge<64>, grid, dim3(256), 0, stream, gp, gate_stride, nkv,
                               seq_lens, max_len, window, Z, ws, op, out_stride);
    }
    return hipGetLastError();
}

}  // namespace qkvf
