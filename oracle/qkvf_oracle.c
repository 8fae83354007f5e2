/*
 * CPU oracle of the decode-batch attention front.  TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the benchmark's CPU-baseline leg call it;
 * the library never does.  It shares no code with the HIP path.
 *
 * What it computes (qkv_front page, module summary; cute_ops page, qkv_front
 * and split_qkv): for 1 <= M <= 16 tokens, the projection
 *     z[m][n] = sum_k x[m][k] * W[n][k]          (K = 8192)
 * rounded to bf16, followed by what the unfused "qknorm + rope + kv insert"
 * op does to that bf16 projection for a bf16 KV cache:
 *   - the output row is [q | k | v | gate], with 8 q heads and 8 gate heads
 *     of 64 columns per KV head and one k and one v head per KV head
 *     (cute_ops page, split_qkv);
 *   - every q and k head gets a weightless RMS norm over its 64 values and
 *     then the interleaved (non-neox) rotary embedding from the fp32 cos|sin
 *     row of the token's position (cute_ops page, unsupported_projection);
 *   - v and gate columns pass through unchanged;
 *   - the token's k and v heads are written into its slot of the paged cache
 *     [pages][num_kv_heads][16][128], K in elements 0..63 and V in 64..127
 *     (cute_ops page, attn2 contract).
 *
 * Arithmetic: the dot products are summed in double in increasing k, the
 * most accurate plain order (the pages allow any fp32 summation order); the
 * norm and the rotation are computed in double and rounded once to bf16.
 * Readings where the pages are silent (the norm's form and epsilon, the
 * cos|sin column layout, negative slots) are listed in the header of each
 * function below.  The file also holds the oracles of the next steps built
 * on the same pages: attn2 (the verify step's paged attention) and
 * LayerFront (the row norm that produces x).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define HIDDEN 8192
#define HEAD_DIM 64
#define PAIRS (HEAD_DIM / 2)
#define QHEADS_PER_KV 8
#define PAGE_SLOTS 16
#define SLOT_WIDTH 128

/* bf16 is the top half of an IEEE binary32. */
double qkvfo_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary32 to bf16, to nearest with ties to even: drop the low 16
 * bits and step the kept part up by one unit when the dropped part is more
 * than half a unit, or exactly half and the kept part is odd.  A carry out of
 * the mantissa moves into the exponent, which is the correct result.
 * Inputs are finite (NaN is not handled). */
uint16_t qkvfo_float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* bf16 of a double: the value goes through binary32 first, as an fp32
 * accumulator or an fp32 epilogue would hold it. */
uint16_t qkvfo_double_to_bf16(double v) { return qkvfo_float_to_bf16((float)v); }

/* Elementwise qkvfo_float_to_bf16 over n values. */
void qkvfo_round_array(const float *in, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = qkvfo_float_to_bf16(in[i]);
}

/*
 * z[m*N + n] = sum over k of x[m][k] * W[n][k], in double, k increasing.
 * abs_sum (optional) receives sum over k of |x[m][k] * W[n][k]|, the scale of
 * any fp32 summation error (used by the tie-aware checker).
 * x: bf16 [M][8192]; W: bf16 [N][8192], both row-major.
 * Rows n are shared out over nthreads OpenMP threads; each output is still
 * one sequential loop over k.
 */
void qkvfo_project(const uint16_t *x, const uint16_t *W, int M, int N,
                   double *z, double *abs_sum, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int n = 0; n < N; ++n) {
        const uint16_t *wrow = W + (size_t)n * HIDDEN;
        for (int m = 0; m < M; ++m) {
            const uint16_t *xrow = x + (size_t)m * HIDDEN;
            double acc = 0.0, mag = 0.0;
            for (int k = 0; k < HIDDEN; ++k) {
                double t = qkvfo_bf16_to_double(xrow[k]) * qkvfo_bf16_to_double(wrow[k]);
                acc += t;
                mag += fabs(t);
            }
            z[(size_t)m * N + n] = acc;
            if (abs_sum)
                abs_sum[(size_t)m * N + n] = mag;
        }
    }
}

/*
 * One q or k head of one token (qkv_front page, module summary: the per-head
 * weightless RMS norm and interleaved RoPE).
 *   p:   the head's 64 bf16 projection values;
 *   cs:  the fp32 cos|sin row of the token's position, cos of pair i in
 *        column i and sin of pair i in column 32 + i, or NULL for a layer
 *        without RoPE (then the head is only normed);
 *   out: the 64 results rounded to bf16; out_d (optional) the same values
 *        before rounding.
 * Norm (reading: mean of squares over the head, epsilon inside the root):
 *   r = 1 / sqrt(sum(p^2) / 64 + eps),  n_c = p_c * r.
 * Rotation of pair i (columns 2i, 2i+1) by (c, s):
 *   o_2i = n_2i * c - n_2i+1 * s,   o_2i+1 = n_2i+1 * c + n_2i * s.
 */
void qkvfo_head(const uint16_t *p, const float *cs, double eps,
                uint16_t *out, double *out_d)
{
    double v[HEAD_DIM];
    double ss = 0.0;
    for (int c = 0; c < HEAD_DIM; ++c) {
        v[c] = qkvfo_bf16_to_double(p[c]);
        ss += v[c] * v[c];
    }
    double r = 1.0 / sqrt(ss / HEAD_DIM + eps);
    for (int c = 0; c < HEAD_DIM; ++c)
        v[c] *= r;
    double o[HEAD_DIM];
    for (int i = 0; i < PAIRS; ++i) {
        double a = v[2 * i], b = v[2 * i + 1];
        if (cs) {
            double c = (double)cs[i], s = (double)cs[PAIRS + i];
            o[2 * i] = a * c - b * s;
            o[2 * i + 1] = b * c + a * s;
        } else {
            o[2 * i] = a;
            o[2 * i + 1] = b;
        }
    }
    for (int c = 0; c < HEAD_DIM; ++c) {
        out[c] = qkvfo_double_to_bf16(o[c]);
        if (out_d)
            out_d[c] = o[c];
    }
}

/*
 * Everything after the projection, for M tokens, on the bf16 projection p
 * [M][N] (N = 1152 * nkv):
 *   y [M][N] bf16: q and k heads normed and rotated, v and gate copied from p
 *   (cute_ops page, split_qkv, for the column blocks);
 *   kv_cache [pages][nkv][16][128] bf16: for token m with slot s >= 0, page
 *   s / 16 and offset s % 16, KV head j gets K = y's k head j in elements
 *   0..63 and V = y's v head j in 64..127 (cute_ops page, attn2 contract);
 *   nothing else in the cache is written.  A negative slot (reading: a padding
 *   token) writes no cache entry.
 * positions index rows of cos_sin [rows][64]; cos_sin NULL means no RoPE.
 */
void qkvfo_epilogue(const uint16_t *p, const int64_t *positions,
                    const int64_t *slots, const float *cos_sin, int nkv,
                    int M, double eps, uint16_t *y, uint16_t *kv_cache)
{
    const int nq = QHEADS_PER_KV * nkv;
    const int N = 2 * (nq + nkv) * HEAD_DIM;
    const int k_col = nq * HEAD_DIM;           /* first k column */
    const int v_col = k_col + nkv * HEAD_DIM;  /* first v column */
    for (int m = 0; m < M; ++m) {
        const uint16_t *prow = p + (size_t)m * N;
        uint16_t *yrow = y + (size_t)m * N;
        const float *cs = cos_sin ? cos_sin + (size_t)positions[m] * HEAD_DIM : NULL;
        memcpy(yrow, prow, (size_t)N * sizeof(uint16_t));
        for (int h = 0; h < nq + nkv; ++h)  /* q heads, then k heads */
            qkvfo_head(prow + h * HEAD_DIM, cs, eps, yrow + h * HEAD_DIM, NULL);
        int64_t s = slots[m];
        if (s < 0)
            continue;
        int64_t page = s / PAGE_SLOTS, off = s % PAGE_SLOTS;
        for (int j = 0; j < nkv; ++j) {
            uint16_t *dst = kv_cache + (((size_t)page * nkv + j) * PAGE_SLOTS + off) * SLOT_WIDTH;
            memcpy(dst, yrow + k_col + j * HEAD_DIM, HEAD_DIM * sizeof(uint16_t));
            memcpy(dst + HEAD_DIM, yrow + v_col + j * HEAD_DIM, HEAD_DIM * sizeof(uint16_t));
        }
    }
}

/*
 * The whole front: projection in double, one rounding to bf16 (through
 * binary32, as an fp32 accumulator holds it), then the epilogue above.
 * z_scratch: caller-provided double [M][N]; p: caller-provided bf16 [M][N]
 * that receives the rounded projection.
 */
void qkvfo_front(const uint16_t *x, const uint16_t *W, const int64_t *positions,
                 const int64_t *slots, const float *cos_sin, int nkv, int M,
                 double eps, double *z_scratch, uint16_t *p, uint16_t *y,
                 uint16_t *kv_cache, int nthreads)
{
    const int N = 2 * (QHEADS_PER_KV * nkv + nkv) * HEAD_DIM;
    qkvfo_project(x, W, M, N, z_scratch, NULL, nthreads);
    for (size_t i = 0; i < (size_t)M * N; ++i)
        p[i] = qkvfo_double_to_bf16(z_scratch[i]);
    qkvfo_epilogue(p, positions, slots, cos_sin, nkv, M, eps, y, kv_cache);
}

/*
 * attn2: paged decode attention of the 8-token verify step, fused with the
 * weightless RMS norm of its output and the sigmoid gate (cute_ops page,
 * attn2 entry: head_dim 64, 8 query heads per KV head, bf16 cache
 * [pages][nkv][16][128] with K | V per slot, 8 query rows per request, any
 * context length L >= 8, optional sliding window).
 *
 * Request r has L = seq_lens[r] tokens; its 8 query rows are the last 8
 * positions, row t at position p = L - 8 + t.  Key position k lives in slot
 * k % 16 of physical page block_table[r * bt_stride + k / 16].  For query
 * head h (KV head h / 8) the row attends keys k in [lo, p] with lo = 0, or
 * lo = max(0, p - window + 1) when window > 0 (readings: causal inside the
 * draft, a window of W keys ending at the row's own position):
 *   s_k  = scale * q . K_k,   a = softmax(s),   o = sum_k a_k V_k,
 *   out  = o / sqrt(mean(o^2) + eps) * sigmoid(gate),  rounded to bf16.
 * q and gate rows are bf16 [R*8][nq*64] with row strides q_stride and
 * gate_stride (elements); out likewise with out_stride.  All in double.
 */
void qkvfo_attn2(const uint16_t *q, int64_t q_stride, const uint16_t *gate,
                 int64_t gate_stride, const uint16_t *kv_cache, int nkv,
                 const int32_t *block_table, int64_t bt_stride,
                 const int32_t *seq_lens, int R, int window, double scale,
                 double eps, uint16_t *out, int64_t out_stride)
{
    const int nq = QHEADS_PER_KV * nkv;
    /* (row, head) pairs are independent; threads only share the loop. */
#pragma omp parallel for schedule(dynamic)
    for (int64_t idx = 0; idx < (int64_t)R * 8 * nq; ++idx) {
        const int r = (int)(idx / (8 * nq));
        const int t = (int)(idx / nq % 8);
        const int h = (int)(idx % nq);
        const int L = seq_lens[r];
        {
            const int64_t row = (int64_t)r * 8 + t;
            const int p = L - 8 + t;
            const int lo = window > 0 ? (p - window + 1 > 0 ? p - window + 1 : 0) : 0;
            {
                const int j = h / QHEADS_PER_KV;
                const uint16_t *qh = q + row * q_stride + (int64_t)h * HEAD_DIM;
                double m = -INFINITY;
                for (int k = lo; k <= p; ++k) {
                    const int32_t page = block_table[(int64_t)r * bt_stride + k / PAGE_SLOTS];
                    const uint16_t *K = kv_cache + (((int64_t)page * nkv + j) * PAGE_SLOTS + k % PAGE_SLOTS) * SLOT_WIDTH;
                    double s = 0.0;
                    for (int d = 0; d < HEAD_DIM; ++d)
                        s += qkvfo_bf16_to_double(qh[d]) * qkvfo_bf16_to_double(K[d]);
                    s *= scale;
                    if (s > m)
                        m = s;
                }
                double l = 0.0, o[HEAD_DIM];
                for (int d = 0; d < HEAD_DIM; ++d)
                    o[d] = 0.0;
                for (int k = lo; k <= p; ++k) {
                    const int32_t page = block_table[(int64_t)r * bt_stride + k / PAGE_SLOTS];
                    const uint16_t *K = kv_cache + (((int64_t)page * nkv + j) * PAGE_SLOTS + k % PAGE_SLOTS) * SLOT_WIDTH;
                    const uint16_t *V = K + HEAD_DIM;
                    double s = 0.0;
                    for (int d = 0; d < HEAD_DIM; ++d)
                        s += qkvfo_bf16_to_double(qh[d]) * qkvfo_bf16_to_double(K[d]);
                    const double a = exp(s * scale - m);
                    l += a;
                    for (int d = 0; d < HEAD_DIM; ++d)
                        o[d] += a * qkvfo_bf16_to_double(V[d]);
                }
                double ss = 0.0;
                for (int d = 0; d < HEAD_DIM; ++d) {
                    o[d] /= l;
                    ss += o[d] * o[d];
                }
                const double rr = 1.0 / sqrt(ss / HEAD_DIM + eps);
                const uint16_t *g = gate + row * gate_stride + (int64_t)h * HEAD_DIM;
                uint16_t *dst = out + row * out_stride + (int64_t)h * HEAD_DIM;
                for (int d = 0; d < HEAD_DIM; ++d) {
                    const double sg = 1.0 / (1.0 + exp(-qkvfo_bf16_to_double(g[d])));
                    dst[d] = qkvfo_double_to_bf16(o[d] * rr * sg);
                }
            }
        }
    }
}

/*
 * LayerFront (layer_front page, class LayerFront and its run method): the
 * first decoder layer's input.  For each of `rows` rows of H = 8192 values:
 *     stream = float(x)                (x bf16 or fp32; exact)
 *     aux    = stream                  (only when aux is not NULL)
 *     out    = bf16(stream * r * w),   r = 1 / sqrt(mean(stream^2) + eps)
 * where the norm is the layer's pre-QKV-projection RMS norm.  Readings (the
 * page names the norm but prints neither its form nor its epsilon): the
 * usual RMS norm over the row with eps inside the root; w is the norm's
 * bf16 weight, or 1 when the norm has none (weight == NULL); the product is
 * rounded once, double -> binary32 -> bf16 as for every other output.
 * x_is_fp32 selects the input type (bf16 bits or fp32 values).  `exact`, when
 * not NULL, receives the double value before rounding (for the checker).
 */
void qkvfo_layer_front(const void *x, int x_is_fp32, int64_t rows, const uint16_t *weight,
                       double eps, float *stream, float *aux, uint16_t *out, double *exact)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float s[HIDDEN];
        for (int k = 0; k < HIDDEN; ++k)
            s[k] = x_is_fp32 ? ((const float *)x)[r * HIDDEN + k]
                             : (float)qkvfo_bf16_to_double(((const uint16_t *)x)[r * HIDDEN + k]);
        double ss = 0.0;
        for (int k = 0; k < HIDDEN; ++k)
            ss += (double)s[k] * (double)s[k];
        const double rr = 1.0 / sqrt(ss / HIDDEN + eps);
        for (int k = 0; k < HIDDEN; ++k) {
            stream[r * HIDDEN + k] = s[k];
            if (aux)
                aux[r * HIDDEN + k] = s[k];
            const double w = weight ? qkvfo_bf16_to_double(weight[k]) : 1.0;
            const double v = (double)s[k] * rr * w;
            if (exact)
                exact[r * HIDDEN + k] = v;
            out[r * HIDDEN + k] = qkvfo_double_to_bf16(v);
        }
    }
}

/*
 * MuseRouting (cute_ops page, MuseRouting entry and class; unsupported_router
 * for the constants): routing of b <= 8 tokens over 256 experts.
 *     score[e] = sigmoid(logit[e])              (fp32)
 *     key[e]   = score[e] + bias[e]             (fp32; the correction bias
 *                                                steers the selection only)
 *     the 8 experts with the largest keys, best first
 *     weight   = score * route_scale / (sum of the 8 scores + 1e-15)
 * Readings (the page names the steps but not their arithmetic): the score
 * is the sigmoid's exact value rounded once to fp32 (computed in double);
 * the key is the fp32 sum; equal keys rank by lower expert id; ids and
 * weights are written best first; the weight is computed in double from the
 * fp32 scores, the 8 scores summed best first, and rounded once to fp32.
 */
#define ROUTE_EXPERTS 256
#define ROUTE_TOP_K 8

float qkvfo_route_score(float logit) { return (float)(1.0 / (1.0 + exp(-(double)logit))); }

void qkvfo_route(const float *logits, int64_t row_stride, const float *bias, double route_scale,
                 int tokens, int32_t *ids, float *weights)
{
    for (int t = 0; t < tokens; ++t) {
        const float *row = logits + (int64_t)t * row_stride;
        float score[ROUTE_EXPERTS], key[ROUTE_EXPERTS];
        int taken[ROUTE_EXPERTS];
        for (int e = 0; e < ROUTE_EXPERTS; ++e) {
            score[e] = qkvfo_route_score(row[e]);
            key[e] = score[e] + bias[e];
            taken[e] = 0;
        }
        int pick[ROUTE_TOP_K];
        for (int k = 0; k < ROUTE_TOP_K; ++k) {
            int best = -1;
            for (int e = 0; e < ROUTE_EXPERTS; ++e)
                if (!taken[e] && (best < 0 || key[e] > key[best]))
                    best = e;      /* strict '>' keeps the lower id on equal keys */
            taken[best] = 1;
            pick[k] = best;
        }
        double sum = 0.0;
        for (int k = 0; k < ROUTE_TOP_K; ++k)
            sum += (double)score[pick[k]];
        for (int k = 0; k < ROUTE_TOP_K; ++k) {
            ids[t * ROUTE_TOP_K + k] = pick[k];
            weights[t * ROUTE_TOP_K + k] =
                (float)((double)score[pick[k]] * route_scale / (sum + 1e-15));
        }
    }
}
