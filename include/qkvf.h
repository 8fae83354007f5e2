/*
 * libqkvfront: the decode-batch attention front on MI355X (gfx950).
 *
 * For 1 <= M <= 16 tokens one call computes, in the order below, what the
 * QKV + o-gate projection followed by the unfused "q/k norm + rope + kv
 * insert" op computes for a bf16 KV cache (qkv_front page, module summary;
 * cute_ops page, qkv_front):
 *   1. p = bf16(x @ W^T): x bf16 [M][8192], W bf16 [N][8192], fp32
 *      accumulation, round to nearest even;
 *   2. on each q and k head (64 columns) of each token: a weightless RMS
 *      norm, n = p / sqrt(mean(p^2) + 1e-6), then the interleaved rotary
 *      embedding of pairs (2i, 2i+1) by the cos|sin row of the token's
 *      position; v and gate columns stay p;
 *   3. the store of the result row y[m] = [q | k | v | gate] (cute_ops page,
 *      split_qkv: per KV head 8 q heads, one k, one v and 8 gate heads, 64
 *      columns each, so N = 1152 * num_kv_heads);
 *   4. the insert of each token's k and v heads into its slot of the paged
 *      cache [pages][num_kv_heads][16][128] bf16, K in elements 0..63 and V
 *      in 64..127 of the slot (cute_ops page, attn2 contract).
 * The result depends only on the launch shape, which is a function of
 * (N, M) alone (qkv_front page, "Structure"): repeated calls are bitwise
 * identical.
 *
 * All pointers are device pointers on the current HIP device.  The caller
 * owns every tensor; the library owns only a small workspace per device
 * (allocated by qkvf_prepare, freed by qkvf_release) through which the
 * kernel's blocks pass their fp32 partial sums.  Every call leaves that
 * workspace as it found it, so no call depends on an earlier one (no
 * counters, no state across calls).  Functions return 0 or a qkvf_status
 * code, never throw and never abort.
 */
#ifndef QKVF_H
#define QKVF_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (the reasons a call is refused: qkv_front page, function
 * "unsupported"; cute_ops page, supports_call and unsupported_projection). */
typedef enum {
    QKVF_OK = 0,
    QKVF_ERR_DEVICE = 1,        /* no current device, not gfx950, or fewer than 256 CUs */
    QKVF_ERR_SHAPE = 2,         /* num_kv_heads not in {1,2,4,8} or N != 1152*num_kv_heads */
    QKVF_ERR_ROWS = 3,          /* M outside [1, 16] */
    QKVF_ERR_ALIGN = 4,         /* a pointer is not aligned as stated below */
    QKVF_ERR_NULLPTR = 5,       /* a required pointer is NULL */
    QKVF_ERR_NOT_PREPARED = 6,  /* no shape bound on this thread, or (N, M) not prepared on this device */
    QKVF_ERR_ALLOC = 7,         /* workspace allocation failed */
    QKVF_ERR_HIP = 8,           /* a HIP runtime call or a launch failed */
    QKVF_ERR_RANGE = 9,         /* qkvf_check: a position or slot out of range, duplicate slots */
    QKVF_ERR_OVERLAP = 10,      /* qkvf_check: an output overlaps another operand */
    QKVF_ERR_MEMORY = 11,       /* qkvf_check: a pointer is not device memory of the current device */
    QKVF_ERR_TIMEOUT = 12       /* qkvf_device_fault: a call gave up waiting for a partial result */
} qkvf_status;

/* Element types of an input that may come in either (qkvf_layer_front). */
typedef enum { QKVF_DTYPE_BF16 = 0, QKVF_DTYPE_F32 = 1 } qkvf_dtype;

/*
 * Prepare the front for N output columns, num_kv_heads KV heads and every
 * row count 1..M on the current device (qkv_front page, function "prepare":
 * ready the variants before graph capture).  Validates the shape, checks the
 * device is gfx950 with room for the kernel's 256 blocks at once (one per
 * CU), allocates and sets up the device workspace once (about 2.4 MB, the
 * same for every shape) and checks on which XCD each block runs (both
 * synchronize the device, once), and binds
 * (N, num_kv_heads) as the calling thread's
 * current shape, which qkvf_run uses.  Call it again to switch shape; it is
 * cheap after the first call.  Not to be called during graph capture.
 * Errors: QKVF_ERR_SHAPE, QKVF_ERR_ROWS, QKVF_ERR_DEVICE, QKVF_ERR_ALLOC.
 */
int qkvf_prepare(int N, int num_kv_heads, int M);

/*
 * Enqueue one front call of M tokens on `stream` for the thread's current
 * shape (qkv_front page, function "launch": the call without the full
 * checks).
 *   x          bf16 [M][8192], row-major, 16-byte aligned (read);
 *   W          bf16 [N][8192], row-major, 16-byte aligned (read);
 *   positions  int64 [M]: row of cos_sin for each token (read);
 *   slots      int64 [M]: cache slot of each token, page = slot / 16,
 *              offset = slot % 16; a negative slot writes no cache entry
 *              (read);
 *   cos_sin    fp32 [rows][64], row p = 32 cos | 32 sin of position p, or
 *              NULL for a layer without RoPE (q and k are then only normed),
 *              16-byte aligned (read);
 *   y          bf16 [M][N], row-major, 16-byte aligned (written; rows >= M
 *              are not touched);
 *   kv_cache   bf16 [pages][num_kv_heads][16][128], 16-byte aligned (only
 *              the M slots named by `slots` are written).
 * The caller guarantees positions < rows of cos_sin, slots < pages * 16,
 * distinct non-negative slots, and no overlap between y, kv_cache and the
 * inputs (qkvf_check verifies all of these).  The call allocates nothing,
 * never synchronizes and only enqueues work on `stream` (so it can be
 * captured in a HIP graph, and replayed any number of times).
 * Ordering: calls on one device share its workspace, so they must not run
 * concurrently (issue them on one stream, or order streams with events).
 * Calls that do overlap are undefined: they can take each other's partial
 * sums and write wrong y and cache entries without any fault being
 * recorded.  Residency: the kernel's 256 blocks (one per CU) wait for each
 * other's partials; other work on the device only delays the blocks that
 * have not started yet.  A block that waits far longer than any call takes
 * (about a second) gives up: it stores no y and no cache entry and records
 * a fault in the device's fault word (qkvf_fault_word, qkvf_device_fault).
 * While the fault word is set, every call on the device stores nothing
 * (y and kv_cache keep their contents), until qkvf_device_fault reports and
 * clears it.
 * Errors (cheap scalar checks only): QKVF_ERR_NOT_PREPARED, QKVF_ERR_ROWS,
 * QKVF_ERR_NULLPTR, QKVF_ERR_ALIGN, QKVF_ERR_DEVICE, QKVF_ERR_HIP.
 */
int qkvf_run(const void *x, const void *W, const int64_t *positions,
             const int64_t *slots, const float *cos_sin, void *y,
             void *kv_cache, int M, hipStream_t stream);

/*
 * qkvf_run for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call and kernel, with N and num_kv_heads given per call, no qkvf_prepare,
 * and the partials passed through the library's static device array instead
 * of a prepared workspace.  The array holds the partials of any call the
 * front accepts (M <= 16, N <= 9216: 2.36 MB per device, kept until the
 * process ends); a larger call is refused (QKVF_ERR_SHAPE, QKVF_ERR_ROWS).
 * It calls no allocating routine.  The first call on a device sets the
 * array up (empties it and checks on which XCD each block runs) and
 * synchronizes the device, so make it before any capture; later calls only
 * enqueue one launch on `stream`.  Every call on a device shares that
 * device's array: calls that overlap on one device race (undefined, as for
 * qkvf_run), so order them on one stream or with events.  Faults behave as
 * for qkvf_run; qkvf_device_fault reports and clears them.  Pointers,
 * layouts and the caller's guarantees are those of qkvf_run.
 * Errors: QKVF_ERR_SHAPE, QKVF_ERR_ROWS, QKVF_ERR_NULLPTR, QKVF_ERR_ALIGN,
 * QKVF_ERR_DEVICE, QKVF_ERR_HIP.
 */
int qkvf_run_static(int N, int num_kv_heads, const void *x, const void *W,
                    const int64_t *positions, const int64_t *slots,
                    const float *cos_sin, void *y, void *kv_cache, int M,
                    hipStream_t stream);

/*
 * Full check of a call before it is launched (qkv_front page, function
 * "unsupported"; cute_ops page, supports_call): shape, rows, alignment,
 * that every pointer is device memory of the current device, that y and
 * kv_cache overlap neither each other nor any input, and, when
 * read_indices != 0, that every position is in [0, table_rows) and every
 * slot is negative or in [0, pages * 16) with no slot repeated.
 * read_indices copies positions and slots to the host and so synchronizes
 * the device; with read_indices == 0 nothing is read from the device.
 * Returns QKVF_OK or the first reason found.  It launches nothing.
 */
int qkvf_check(int N, int num_kv_heads, int M, int64_t pages,
               int64_t table_rows, const void *x, const void *W,
               const int64_t *positions, const int64_t *slots,
               const float *cos_sin, const void *y, const void *kv_cache,
               int read_indices);

/* Static text for a status code (never NULL). */
const char *qkvf_strerror(int status);

/*
 * The launch shape of (N, M): grid blocks of the projection kernel, the
 * split of K across blocks, waves per block and the most tiles of up to 16 W
 * rows a block owns.  With 4 or 8 KV heads each XCD owns whole heads, heads
 * x * H / 8 .. (x + 1) * H / 8 - 1 of the H = N / 64, and its 32 blocks share
 * their tiles equally.  With 1 or 2 KV heads each XCD owns N / 8 rows (whole
 * q and k heads, then v and gate rows) and every block an equal share of
 * them, as one short tile and 16-row tiles: 36 rows in 3 tiles with 1 KV
 * head, and with 2 KV heads 72 rows in 5 tiles (8 K splits) from 12 token
 * rows, 36 rows in 3 tiles (4 K splits, 2048 K each) below.
 * A pure function of its arguments.  Returns QKVF_OK, QKVF_ERR_SHAPE or
 * QKVF_ERR_ROWS.  Any output pointer may be NULL.
 */
int qkvf_plan(int N, int M, int *grid, int *k_splits, int *waves_per_block,
              int *tiles_per_block);

/* Bytes of the device workspace qkvf_prepare allocates per device. */
size_t qkvf_workspace_bytes(void);

/*
 * How the kernel's blocks hand partial sums to each other.  mode 0 (the
 * default): a partial read on the XCD that produced it is stored plainly and
 * read from that XCD's L2, when qkvf_prepare found that the device places a
 * kernel's blocks on its 8 XCDs round robin (checked once per device with a
 * small kernel; if not, mode 1 is used).  mode 1: every partial is written
 * through to memory.
 * Both modes give bitwise the same results; mode 1 is a little slower.  For
 * diagnostics and tests; applies to calls launched afterwards, process-wide.
 * Returns QKVF_OK, or QKVF_ERR_RANGE for another mode.
 */
int qkvf_set_handoff(int mode);

/*
 * For tests of the failure path: the polling rounds a block of a later
 * qkvf_run waits for another block's partials before it gives up (stores
 * nothing for its part and records a fault).  rounds == 0 restores the
 * default (about a second); 1 gives up at the first round that finds a
 * partial missing.  Process-wide.  Returns QKVF_OK.
 */
int qkvf_set_spin_limit(unsigned rounds);

/*
 * Synchronize the current device and report whether any call on it since the
 * last query gave up waiting for a partial result (QKVF_ERR_TIMEOUT; that
 * call's missing outputs and every later call's outputs were not written).
 * Clears the fault and sets the workspace up again, so calls work again.
 * Returns QKVF_OK when no call failed (or nothing was prepared on the
 * device), QKVF_ERR_DEVICE when there is no current HIP device, QKVF_ERR_HIP
 * on a runtime error.
 */
int qkvf_device_fault(void);

/*
 * The device address of the current device's fault word (unsigned, 4-byte
 * aligned, owned by the library until qkvf_release): 0 while every call has
 * completed, nonzero once a call gave up waiting.  A caller can copy it on
 * its own stream after its calls, without synchronizing the device; only
 * qkvf_device_fault clears it.  Errors: QKVF_ERR_NULLPTR (word == NULL),
 * QKVF_ERR_DEVICE, QKVF_ERR_NOT_PREPARED (no workspace on this device).
 */
int qkvf_fault_word(unsigned **word);

/*
 * attn2: paged decode attention of the 8-token verify step fused with the
 * weightless RMS norm of its output and the sigmoid gate, the input of the
 * layer's o_proj (cute_ops page, attn2 entry).  Per request r with
 * L = seq_lens[r] >= 8 tokens, query row t (0..7, row index 8 r + t) sits at
 * position L - 8 + t; for each q head h (KV head h / 8) it attends the keys
 * at positions lo .. L - 8 + t (lo = 0, or L - 8 + t - window + 1 clamped to
 * 0 with a sliding window), whose K | V sit in slot k % 16 of physical page
 * block_table[r * block_table_stride + k / 16] of the cache that
 * qkvf_run fills.  With s = q K^T / 8 (softmax scale 1/sqrt(64)) and
 * o = softmax(s) V, the output is o / sqrt(mean(o^2) + 1e-6) *
 * sigmoid(gate), per head of 64 values, rounded to bf16.
 *
 * qkvf_attn2_prepare binds a layer's (num_kv_heads, max_model_len,
 * max_reqs, window) to the calling thread (window 0: none; a window of at
 * least max_model_len is none) and sizes the device workspace in which
 * calls split their keys over several blocks (the launch shape depends on
 * these values and the call's request count only, see qkvf_attn2_plan, so
 * it is fixed for a batch size and capturable; qkvf_attn2_prepare_ex can
 * fix each request's split count for every batch size).  It may
 * allocate; a workspace it outgrows stays allocated (a call already
 * launched may still use it) until qkvf_release.
 * Errors: QKVF_ERR_SHAPE, QKVF_ERR_ROWS (max_reqs outside [1, 64]),
 * QKVF_ERR_DEVICE, QKVF_ERR_ALLOC.
 */
int qkvf_attn2_prepare(int num_kv_heads, int max_model_len, int max_reqs, int window);

/*
 * qkvf_attn2_prepare with a choice of split count.  batch_invariant == 0 is
 * qkvf_attn2_prepare: the requests of a call share its split slots (about
 * 256 blocks per launch) in proportion to their lengths, so a request's
 * output may differ in its last bits (the fp32 summation order of its
 * splits) with the requests it is batched with.  batch_invariant == 1: every
 * request takes the split count of one request alone (qkvf_attn2_plan with
 * num_reqs = 1), so a request's output bits depend only on its own inputs
 * and the layer; a batch of R requests then launches R times that many
 * blocks and sizes the workspace for it (R x the partials of one request).
 * Errors: those of qkvf_attn2_prepare, and QKVF_ERR_RANGE for another
 * batch_invariant value.
 */
int qkvf_attn2_prepare_ex(int num_kv_heads, int max_model_len, int max_reqs, int window,
                          int batch_invariant);

/*
 * Enqueue attn2 for num_reqs requests on `stream` (device pointers):
 *   q         bf16 rows [8 num_reqs][>= 512 nkv] with row stride
 *             q_row_stride elements: the q columns (for the front's output y,
 *             q = y, stride N), 16-byte aligned, stride a multiple of 8;
 *   gate      bf16 rows, the gate columns (y + 1152 nkv - 512 nkv for y), row
 *             stride gate_row_stride (8-byte aligned, multiple of 4);
 *   kv_cache  bf16 [pages][num_kv_heads][16][128], 16-byte aligned;
 *   block_table int32 [num_reqs][block_table_stride] physical page numbers,
 *             at least ceil(seq_lens[r] / 16) of them in row r;
 *   seq_lens  int32 [num_reqs], each in [8, max_model_len] (the kernel clamps
 *             a length outside that range, giving a meaningless result);
 *   out       bf16 rows [8 num_reqs][512 nkv], row stride out_row_stride
 *             (8-byte aligned, multiple of 4), written.
 * The caller guarantees page numbers below the cache's page count and finite
 * cache entries at the positions a row attends.  Allocates
 * nothing, never synchronizes; calls on one device share its workspace and
 * must be ordered.  Errors: QKVF_ERR_NOT_PREPARED, QKVF_ERR_ROWS,
 * QKVF_ERR_NULLPTR, QKVF_ERR_SHAPE (a stride too small), QKVF_ERR_ALIGN,
 * QKVF_ERR_DEVICE, QKVF_ERR_HIP.
 */
int qkvf_attn2_run(const void *q, int64_t q_row_stride, const void *gate,
                   int64_t gate_row_stride, const void *kv_cache,
                   const int32_t *block_table, int64_t block_table_stride,
                   const int32_t *seq_lens, int num_reqs, void *out,
                   int64_t out_row_stride, hipStream_t stream);

/* The split slots per KV head of an attn2 launch for a layer and a request
 * count: ceil(256 / num_kv_heads) (about one 16-wave block per CU), capped
 * by num_reqs times the splits one request can take (one per 128 keys of the
 * span its rows attend, max_model_len or window + 7, and at most 64); 1 when
 * that is not more than num_reqs, meaning every request takes one split and
 * there is no merge pass.  The requests of a call share the slots: one split
 * length for the call, the shortest whole number of 128-key steps for which
 * every request's splits fit, so a request's split count follows its length.
 * With num_reqs = 1 it is the request's split count, which batch-invariant
 * splits use for every request.  A pure function of its arguments.
 * Returns QKVF_OK, QKVF_ERR_SHAPE or QKVF_ERR_ROWS. */
int qkvf_attn2_plan(int num_kv_heads, int max_model_len, int window, int num_reqs,
                    int *splits);

/*
 * LayerFront: the first decoder layer's input (layer_front page, class
 * LayerFront, method run).  For each of `rows` rows of 8192 values:
 *     stream = float(x)                    the fp32 residual stream
 *     aux    = stream                      only when aux != NULL (an aux layer)
 *     out    = bf16(stream * r * w),       r = 1 / sqrt(mean(stream^2) + eps)
 * the layer's pre-QKV-projection RMS norm, whose output is the front's x.
 * w is the norm's bf16 weight [8192], or 1 when weight == NULL (a weightless
 * norm).  eps is the norm's epsilon (>= 0, finite).  Device pointers:
 *   x       [rows][8192] of x_dtype (QKVF_DTYPE_BF16 or QKVF_DTYPE_F32),
 *           16-byte (bf16) or 32-byte (fp32) aligned, contiguous rows;
 *   stream  fp32 [rows][8192], 32-byte aligned, written; with an fp32 x it
 *           may be x itself (updated in place);
 *   aux     fp32 [rows][8192], 32-byte aligned, written, or NULL;
 *   out     bf16 [rows][8192], 16-byte aligned, written;
 *   weight  bf16 [8192], 16-byte aligned, or NULL.
 * Apart from stream == x, outputs must not overlap each other or the inputs.
 * rows == 0 does nothing.  One launch on `hip_stream`; allocates nothing and
 * never synchronizes (graph-capturable).  Errors: QKVF_ERR_SHAPE (x_dtype or
 * eps), QKVF_ERR_ROWS (rows < 0 or > 2^20), QKVF_ERR_NULLPTR, QKVF_ERR_ALIGN,
 * QKVF_ERR_DEVICE (not a gfx950), QKVF_ERR_HIP.
 */
int qkvf_layer_front(const void *x, int x_dtype, int64_t rows, const void *weight, float eps,
                     float *stream, float *aux, void *out, hipStream_t hip_stream);

/*
 * MuseRouting: the routing of one MoE layer for decode batches of 1 to 8
 * tokens (cute_ops page, MuseRouting entry and class; unsupported_router for
 * the constants: sigmoid scores, top-8 of 256 experts, division epsilon
 * 1e-15).  For each token t:
 *     score[e] = sigmoid(logits[t][e])        fp32, the exact sigmoid rounded once
 *     key[e]   = score[e] + bias[e]           fp32 (the correction bias steers the
 *                                             selection only)
 *     ids[t]   = the 8 experts with the largest keys, best first; equal keys
 *                rank by lower expert id
 *     weights[t][k] = score[ids[t][k]] * route_scale / (sum of the 8 scores + 1e-15)
 *                computed in double (the scores summed best first), rounded once
 *                to fp32.
 * The router's output multiplier must already be folded into its weight, so
 * the logits are final.  Device pointers: logits fp32 [num_tokens] rows of
 * >= 256 values, row stride logits_row_stride elements (a multiple of 4, so
 * every row is 16-byte aligned), 16-byte aligned; bias fp32 [256], 16-byte
 * aligned; ids int32 [num_tokens][8] and weights fp32 [num_tokens][8],
 * 4-byte aligned, written.  Logits and bias must be finite.  One launch on
 * `stream`; allocates nothing, never synchronizes (graph-capturable).  The
 * routing metadata for other systems' MoE GEMMs is not produced.
 * Errors: QKVF_ERR_ROWS (num_tokens outside [1, 8]), QKVF_ERR_SHAPE (row
 * stride below 256, route_scale not finite), QKVF_ERR_NULLPTR,
 * QKVF_ERR_ALIGN, QKVF_ERR_DEVICE, QKVF_ERR_HIP.
 */
int qkvf_route(const float *logits, int64_t logits_row_stride, const float *bias,
               double route_scale, int num_tokens, int32_t *ids, float *weights,
               hipStream_t stream);

/*
 * A plain streaming read, measurement context for the front's roofline (not
 * a step of the method): how fast the current device streams `bytes` of
 * device memory with the front's launch shape (256 blocks of 512 threads)
 * and load shape (non-temporal 16-byte loads), 16 in flight per lane.  Block
 * b reads the b-th 1/256 of src; thread t of it reads 16-byte pieces t,
 * t + 512, ... of that share and stores the XOR of their 32-bit words in
 * sink[512 b + t].
 *   src   device memory, 16-byte aligned, bytes a whole multiple of 2 MiB
 *         (256 * 512 * 16), at most 128 GiB (read);
 *   sink  device memory, unsigned [256 * 512], 4-byte aligned (written).
 * One launch on `stream`; allocates nothing, never synchronizes.
 * Errors: QKVF_ERR_NULLPTR, QKVF_ERR_SHAPE (bytes not a positive multiple
 * of 2 MiB, or too large), QKVF_ERR_ALIGN, QKVF_ERR_DEVICE, QKVF_ERR_HIP.
 */
int qkvf_stream_read(const void *src, size_t bytes, unsigned *sink, hipStream_t stream);

/* Synchronize each device that holds a workspace, free every workspace of
 * the library and forget prepared shapes.  No call may be made concurrently
 * from another thread. */
void qkvf_release(void);

#ifdef __cplusplus
}
#endif

#endif /* QKVF_H */
