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
// q heads 2w, 2w + 1 (16 rows, row c = 8 (h - 2w) + t).  Keys stream in
// chunks of 32 (two pages of 16 slots), staged in LDS as K [32 keys][64]
// (16-byte chunks XOR-swizzled by key) and V^T [64][32 keys]:
//   S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, A = 16 keys, B = 16 query rows;
//                 lane l holds query l % 16 and keys 4 (l / 16) + v),
//   online softmax per query (max over the lane's 8 keys, then across the 4
//                 lane groups holding the same query),
//   O^T += V^T P^T (A = 16 dims x the lane group's 8 keys, B = the lane's 8
//                 probabilities as bf16 hi + lo parts, so no lane exchange is
//                 needed and the weights keep ~16 bits).
// With one split the block finishes the rows itself; otherwise it writes its
// (max, sum, O) per row to the workspace and attn2_merge combines the splits
// in split order, then applies the norm and the gate.
#include <hip/hip_runtime.h>

#include "qkvf_internal.h"

namespace qkvf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32;                     // keys per step (two pages)
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float sigmoidf(float g) { return 1.f / (1.f + __expf(-g)); }

// Key range [first, end) of split z for request length L; empty if first >= end.
__device__ inline void split_range(int L, int window, int Z, int z, int *first, int *end)
{
    const int lo = window > 0 ? max(0, L - 8 - window + 1) : 0;
    const int base = lo & ~(kPageSlots - 1);            // page aligned
    const int chunks = (L - base + kChunk - 1) / kChunk;
    const int per = (chunks + Z - 1) / Z;
    const int c0 = min(chunks, z * per), c1 = min(chunks, (z + 1) * per);
    *first = base + c0 * kChunk;
    *end = min(L, base + c1 * kChunk);
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
    const int lo0 = window > 0 ? max(0, L - 8 - window + 1) : 0;   // earliest key of any row
    const float sc = 0.125f * kLog2e;          // softmax scale, in log2 units

    int first, end;
    split_range(L, window, Z, z, &first, &end);

    // Q^T operand: lane (c, g) holds q[row][head][32 s + 8 g .. + 7], s = 0, 1.
    const __bf16 *qrow = q + row * q_stride + int64_t(head) * kHeadDim;
    const bf16x8 qv0 = *reinterpret_cast<const bf16x8 *>(qrow + 8 * g);
    const bf16x8 qv1 = *reinterpret_cast<const bf16x8 *>(qrow + 32 + 8 * g);

    // Staging: the chunk's two pages are 512 pieces of 16 bytes; thread tid
    // moves pieces tid and tid + 256: page p = piece / 256, slot = (piece %
    // 256) / 16, part = piece % 16 (0-7: K dims 8 part.., 8-15: V dims).
    auto load_chunk = [&](int k0, bf16x8 *piece) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pc = tid + 256 * i;
            const int key = k0 + (pc >> 8) * kPageSlots + ((pc & 255) >> 4);
            if (key < end && key >= lo0) {
                const int page = block_table[int64_t(r) * bt_stride + key / kPageSlots];
                const __bf16 *src = kv_cache +
                    ((int64_t(page) * nkv + j) * kPageSlots + key % kPageSlots) * kSlotWidth +
                    (pc & 15) * 8;
                piece[i] = *reinterpret_cast<const bf16x8 *>(src);
            } else {
                piece[i] = bf16x8{};
            }
        }
    };
    auto stage_chunk = [&](int buf, const bf16x8 *piece) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pc = tid + 256 * i;
            const int key = (pc >> 8) * kPageSlots + ((pc & 255) >> 4);  // 0..31
            const int part = pc & 15;
            if (part < 8) {
                *reinterpret_cast<bf16x8 *>(&Ks[buf][key * kHeadDim + 8 * (part ^ (key & 7))]) =
                    piece[i];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    Vt[buf][(8 * (part - 8) + e) * kChunk + key] = piece[i][e];
            }
        }
    };

    float m = -INFINITY;   // running max of this lane's query (log2 units)
    float l = 0.f;         // this lane's part of the running sum
    f32x4 o[4] = {};       // O^T[16 dt + 4 g + v][c]

    bf16x8 piece[2];
    int k0 = first;
    if (k0 < end)
        load_chunk(k0, piece);
    int buf = 0;
    for (; k0 < end; k0 += kChunk, buf ^= 1) {
        stage_chunk(buf, piece);
        if (k0 + kChunk < end)
            load_chunk(k0 + kChunk, piece);
        __syncthreads();

        // S^T for 32 keys: two key tiles of 16.
        f32x4 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int key = 16 * kt + c;  // A row = lane % 16
            const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                &Ks[buf][key * kHeadDim + 8 * ((g) ^ (key & 7))]);
            const bf16x8 kb = *reinterpret_cast<const bf16x8 *>(
                &Ks[buf][key * kHeadDim + 8 * ((4 + g) ^ (key & 7))]);
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv0, a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qv1, a, 0, 0, 0);
            s[kt] = a;
        }
        // Mask and scale; lane holds keys k0 + 16 kt + 4 g + v of query c.
        float mc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int kp = k0 + 16 * kt + 4 * g + v;
                const bool ok = kp >= lo && kp <= pos && kp < end;
                s[kt][v] = ok ? s[kt][v] * sc : -INFINITY;
                mc = fmaxf(mc, s[kt][v]);
            }
        mc = fmaxf(mc, __shfl_xor(mc, 16, 64));
        mc = fmaxf(mc, __shfl_xor(mc, 32, 64));
        const float mn = fmaxf(m, mc);
        // alpha rescales the old state; with nothing seen yet it is 0.
        const float alpha = mn == -INFINITY ? 1.f : exp2f(m - mn);
        // Each weight goes in as bf16 hi + lo parts (two products), so the
        // weights keep about 16 bits rather than bf16's 8.
        bf16x8 ph, pl;
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float e = mn == -INFINITY ? 0.f : exp2f(s[kt][v] - mn);
                ps += e;
                const __bf16 hi = __bf16(e);
                ph[4 * kt + v] = hi;
                pl[4 * kt + v] = __bf16(e - float(hi));
            }
        l = l * alpha + ps;
        m = mn;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            o[dt] *= alpha;
            // V^T rows 16 dt + c (A row = lane % 16), keys 4 g .. and 16 + 4 g ..
            const int d = 16 * dt + c;
            const bf16x4 va = *reinterpret_cast<const bf16x4 *>(&Vt[buf][d * kChunk + 4 * g]);
            const bf16x4 vb = *reinterpret_cast<const bf16x4 *>(&Vt[buf][d * kChunk + 16 + 4 * g]);
            const bf16x8 vv = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, ph, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pl, o[dt], 0, 0, 0);
        }
        __syncthreads();  // the next chunk reuses this buffer two steps later
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

// Merge the Z partials of each row in split order, then the norm and gate.
// One block per (KV head, request); 16 threads per row, 4 dims each.
__global__ void __launch_bounds__(256)
attn2_merge(const __bf16 *__restrict__ gate, int64_t gate_stride, int nkv, int Z,
            const float *__restrict__ ws, __bf16 *__restrict__ out, int64_t out_stride)
{
    const int j = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int d0 = 4 * (tid & 15);
#pragma unroll 1
    for (int rr0 = 0; rr0 < 64; rr0 += 16) {
        const int qr = rr0 + (tid >> 4);      // row 8 hh + t
        const int hh = qr >> 3, t = qr & 7;
        const float *src = ws + ((int64_t(r) * nkv + j) * Z * 64 + qr) * kAttn2PartialFloats;
        const int64_t zstride = int64_t(64) * kAttn2PartialFloats;
        float M = -INFINITY;
        for (int zz = 0; zz < Z; ++zz)
            M = fmaxf(M, src[zz * zstride]);
        float lsum = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int zz = 0; zz < Z; ++zz) {
            const float mz = src[zz * zstride];
            const float w = mz == -INFINITY ? 0.f : exp2f(mz - M);
            lsum += w * src[zz * zstride + 1];
            const f32x4 oz = *reinterpret_cast<const f32x4 *>(src + zz * zstride + 4 + d0);
            acc += w * oz;
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        acc *= inv;
        float ss = acc[0] * acc[0] + acc[1] * acc[1] + acc[2] * acc[2] + acc[3] * acc[3];
#pragma unroll
        for (int k = 1; k < 16; k <<= 1)
            ss += __shfl_xor(ss, k, 64);
        const float rrs = rsqrtf(ss * (1.f / kHeadDim) + kAttn2Eps);
        const int64_t row = int64_t(r) * 8 + t;
        const int head = kQPerKv * j + hh;
        const bf16x4 gv = *reinterpret_cast<const bf16x4 *>(gate + row * gate_stride + head * kHeadDim + d0);
        bf16x4 res;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            res[v] = __bf16(acc[v] * rrs * sigmoidf(float(gv[v])));
        *reinterpret_cast<bf16x4 *>(out + row * out_stride + head * kHeadDim + d0) = res;
    }
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
    if (Z > 1)
        hipLaunchKernelGGL(attn2_merge, dim3(nkv, R), dim3(256), 0, stream,
                           static_cast<const __bf16 *>(gate), gate_stride, nkv, Z, ws,
                           static_cast<__bf16 *>(out), out_stride);
    return hipGetLastError();
}

}  // namespace qkvf
