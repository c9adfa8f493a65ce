/*
 * infini_attn.h -- C ABI of the Infini-attention block on gfx950: forward,
 * streaming decode step, backward pass, and the block with its input and
 * output projections.
 *
 * The operation ("Infini-Attention" (AI Wiki), sections "What happens inside
 * the Infini-attention block?" and "How does the compressive memory work?";
 * "Hugging Face Infini-Attention Reproduction Analysis", section
 * "Infini-Attention Mechanism", steps 1-6):
 *
 *   the length-L stream is cut into segments of seg_len tokens (the last one
 *   may be shorter); for segment s, with Q_s, K_s, V_s its rows and (M, z) the
 *   state left by segment s-1,
 *     A_dot = causal softmax(Q_s K_s^T / sqrt(d)) V_s        (inside the segment)
 *     A_mem = sigma(Q_s) M / (sigma(Q_s) z)                   (one scalar per row)
 *     out_s = sigmoid(beta_h) A_mem + (1 - sigmoid(beta_h)) A_dot
 *   then the state absorbs the segment:
 *     linear: M += sigma(K_s)^T V_s
 *     delta:  M += sigma(K_s)^T (V_s - sigma(K_s) M / (sigma(K_s) z))
 *     both:   z += sum_t sigma(K_s,t)
 *   with sigma(x) = ELU(x) + 1 = (x > 0 ? x + 1 : exp(x)). Retrieval and the
 *   delta prediction both read the state from before the segment. Only (M, z)
 *   crosses a segment boundary.
 *
 * Readings of what the pages leave open: the softmax scale is 1/sqrt(d) with d
 * the head width; there is one (M, z) per (batch element, KV head) with M of
 * shape (d, d), and grouped query heads h read the memory of KV head
 * h / (Hq / Hkv); the causal mask keeps the diagonal; sigma applies to the
 * unscaled Q and K; no epsilon is added to any denominator (z0 > 0 makes them
 * positive).
 *
 * Layouts (all row-major, contiguous, device memory):
 *   q, out      [B][Hq][L][d]      element type `dtype`
 *   k, v        [B][Hkv][L][d]     element type `dtype`
 *   beta        [Hq]               float (raw beta; the sigmoid is applied inside)
 *   M0, M_final [B][Hkv][d][d]     float, M[key dim][value dim]
 *   z0, z_final [B][Hkv][d]        float, every entry > 0 (not checked)
 *
 * Ownership: the caller owns every buffer, including the workspace; the
 * library allocates no device memory. Calls on different streams with
 * different workspaces may run concurrently. `out` must not overlap any
 * input. M_final may be M0 and z_final may be z0 (an in-place carry); any
 * other overlap is rejected.
 *
 * Streams: a forward call with more than one segment, a workspace of the
 * full size (infini_attn_workspace_size) and a memory scan in the direct form
 * (seg_len < d, or d_key != d_value), or the linear rule's affine form over
 * at least 64 segments, on a large call (B*Hq*L*d >= 2^26) starts the
 * attention of segment 0 at once and runs the scan of the later
 * segments on an auxiliary stream beside it, in two windows, each window's
 * attention on `stream` waiting for its own window's scan (events). Every
 * other call runs on `stream` alone: each window's scan, then its attention.
 * The auxiliary stream (default priority) and its five events are created
 * once per device, on the first such call with that device current, and kept
 * until the process ends; `stream` must belong to the current device. The
 * call returns with every output ordered before `stream`'s later work, as if
 * all of it ran on `stream`; calls that use the auxiliary stream enqueue one
 * at a time (a host mutex), and their scans share it. Results are the same
 * bit for bit whichever plan runs.
 *
 * Errors: every check runs on the host before anything is enqueued; on an
 * error nothing is written and nothing launches. Execution is asynchronous on
 * `stream`: a fault inside a kernel surfaces at the caller's next
 * synchronisation. NaN or Inf inputs are not checked; they stay inside the
 * (batch, head) slices they touch.
 */
#ifndef INFINI_ATTN_H
#define INFINI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Memory update rule ("How does the compressive memory work?"). */
typedef enum {
  INFINI_RULE_LINEAR = 0, /* M += sigma(K)^T V (the additive variant) */
  INFINI_RULE_DELTA = 1   /* M += sigma(K)^T (V - sigma(K) M / (sigma(K) z)) */
} infini_rule_t;

/* Element type of q, k, v and out. The state is always float. */
typedef enum {
  INFINI_F32 = 0,  /* float in and out; every product in float */
  INFINI_BF16 = 1  /* bfloat16 in and out; bf16 MFMA operands, float accumulation */
} infini_dtype_t;

typedef enum {
  INFINI_OK = 0,
  INFINI_ERR_INVALID_ARG = 1, /* a size < 1, Hq % Hkv != 0, a null pointer, a bad enum, a forbidden overlap */
  INFINI_ERR_UNSUPPORTED = 2, /* d not in {32, 64, 128}; decode: Hq / Hkv > 16 or seg_len > 16384 */
  INFINI_ERR_MISALIGNED = 3,  /* a pointer not 16-byte aligned */
  INFINI_ERR_WORKSPACE = 4,   /* workspace smaller than infini_attn_workspace_size's minimum */
  INFINI_ERR_HIP = 5          /* the HIP runtime refused a launch or a copy */
} infini_status_t;

/*
 * Workspace sizes of a forward call with these sizes, in bytes.
 *   *full_bytes: enough to process every segment in one pass, with the scan
 *                beside the attention (see Streams above);
 *   *min_bytes:  the least the call accepts; it then walks the segments in
 *                windows that fit, which adds launches but gives the same
 *                result bit for bit.
 * Pure host function; touches no device. Either output pointer may be NULL.
 * Returns INFINI_ERR_INVALID_ARG / INFINI_ERR_UNSUPPORTED for sizes that
 * infini_attn_forward would reject.
 */
infini_status_t infini_attn_workspace_size(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype, size_t* full_bytes, size_t* min_bytes);

/*
 * The block forward: out, M_final, z_final from q, k, v, beta, M0, z0.
 *   B, Hq, Hkv, L, d, seg_len: sizes (all >= 1, Hq % Hkv == 0, d in {32, 64, 128});
 *   rule: an infini_rule_t; dtype: an infini_dtype_t;
 *   q, k, v, beta, M0, z0: inputs (device pointers, layouts above);
 *   out, M_final, z_final: outputs (device pointers, layouts above);
 *   workspace, workspace_bytes: caller-owned device scratch (256-byte aligned
 *     recommended, 16 required), at least the minimum size above;
 *   stream: a hipStream_t, or NULL for the null stream.
 * Returns INFINI_OK once every kernel is enqueued.
 */
infini_status_t infini_attn_forward(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    void* out, float* M_final, float* z_final,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory or hold a workspace (code
 * under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc): infini_attn_forward with its workspace replaced by a scratch
 * array of INFINI_NOALLOC_SCRATCH_BYTES (64 MiB) that the library keeps in
 * each GPU's memory, a static device array present from the library's first
 * use of that GPU until the process ends.
 *   Arguments, layouts, overlaps and results as infini_attn_forward, without
 *   the workspace; the output is the same bit for bit. It always runs on
 *   `stream` alone (the serial plan, no auxiliary stream) and calls no
 *   hipMalloc, hipFree or other allocating routine. The first call on a
 *   device looks up the array's address (hipGetSymbolAddress) with that
 *   device current and keeps it; make that first call outside graph capture.
 *   Errors as infini_attn_forward, and INFINI_ERR_WORKSPACE when the call's
 *   minimum workspace (min_bytes of infini_attn_workspace_size) exceeds
 *   INFINI_NOALLOC_SCRATCH_BYTES (a full-size workspace beyond it only means
 *   more windows); INFINI_ERR_HIP when the array's address cannot be had.
 *   Concurrency: all calls on one GPU share that GPU's one array, which keeps
 *   the last call's contents (nothing in it needs to start at zero). Calls on
 *   one stream run one after another; calls that can run at the same time on
 *   one GPU (different streams, graphs replayed concurrently) race on the
 *   array and give wrong results.
 */
#define INFINI_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
infini_status_t infini_attn_forward_noalloc(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    void* out, float* M_final, float* z_final, void* stream);

/*
 * The forward with a key width different from the value width
 * ("Infini-Attention" (AI Wiki), "How does the compressive memory work?": the
 * memory M maps d_key-dimensional features to d_value-dimensional values).
 * Identical to infini_attn_forward when d_key == d_value (the same call).
 *   q        [B][Hq][L][d_key]     k [B][Hkv][L][d_key]    element type
 *   v        [B][Hkv][L][d_value]  out [B][Hq][L][d_value] element type
 *   M0, M_final [B][Hkv][d_key][d_value] float; z0, z_final [B][Hkv][d_key]
 * The softmax scale is 1/sqrt(d_key). d_key and d_value are each 32, 64 or
 * 128 (else INFINI_ERR_UNSUPPORTED). With d_key != d_value the memory runs as
 * the segment-by-segment scan (not the affine form); numerics as
 * infini_attn_forward. Workspace sizes
 * from infini_attn_workspace_size_kv, with the same full and minimum
 * meanings; arguments, overlaps and errors as infini_attn_forward.
 */
infini_status_t infini_attn_workspace_size_kv(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d_key, int64_t d_value,
    int64_t seg_len, int32_t rule, int32_t dtype, size_t* full_bytes, size_t* min_bytes);
infini_status_t infini_attn_forward_kv(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d_key, int64_t d_value,
    int64_t seg_len, int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    void* out, float* M_final, float* z_final,
    void* workspace, size_t workspace_bytes, void* stream);
/* infini_attn_forward_kv with the events of infini_attn_forward_timed. */
infini_status_t infini_attn_forward_kv_timed(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d_key, int64_t d_value,
    int64_t seg_len, int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    void* out, float* M_final, float* z_final,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

/*
 * infini_attn_forward, plus HIP events recorded on `stream`, for timing its
 * phases:
 *   events[0] at the start of the call;
 *   events[1] when the first attention kernel may start (after the first
 *             window's memory scan: the part of the scan on the critical path);
 *   events[2] after the last attention kernel (the later windows' scans run
 *             beside the attention on the auxiliary stream, or between the
 *             attention kernels on `stream` when the workspace holds only one
 *             segment's data).
 * Indices from n_events on are not recorded (at most 3 are used). `events`
 * holds hipEvent_t handles the caller created (as void*); none may be NULL.
 * Everything else is as in infini_attn_forward.
 */
infini_status_t infini_attn_forward_timed(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    void* out, float* M_final, float* z_final,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

/*
 * Streaming decode ("Infini-Attention" (AI Wiki), "Why is the memory
 * footprint bounded?": a stream runs segment by segment with only (M, z)
 * carried, so the work per token is bounded by seg_len; the per-token
 * arithmetic is the forward's, "What happens inside the Infini-attention
 * block?").
 *
 * One call takes one new token for every (batch element, head): the token at
 * position `pos` (0 <= pos < seg_len) of its segment. It
 *   1. writes the token's key and value into row `pos` of the caches;
 *   2. computes, for every query head h, the forward's output for this token:
 *      causal softmax over cache rows 0..pos (this segment's tokens so far,
 *      the new one included), retrieval sigma(q) M / (sigma(q) z) from (M, z)
 *      as passed (the state before the segment), and the sigmoid(beta_h) gate;
 *   3. when pos == seg_len - 1 (the segment is complete), folds cache rows
 *      0..seg_len-1 into (M, z) in place with the update rule.
 * Decoding a stream token by token, with pos = t mod seg_len and the same
 * caches and state passed each time, gives the outputs of infini_attn_forward
 * on the stream and, after each full segment, its state (up to rounding: the
 * retrieval here reads the float state, the forward a snapshot in the element
 * type). The caller keeps `pos`; cache rows pos+1.. are neither read nor
 * written.
 *
 * Layouts (row-major, contiguous, device memory):
 *   q, out            [B][Hq][d]            element type `dtype`
 *   k, v              [B][Hkv][d]           element type `dtype`
 *   beta              [Hq]                  float
 *   k_cache, v_cache  [B][Hkv][seg_len][d]  element type `dtype`; read and written
 *   M, z              [B][Hkv][d][d], [B][Hkv][d]  float; read, and written at a segment end
 * Sizes as for the forward, plus Hq / Hkv <= 16 and seg_len <= 16384
 * (INFINI_ERR_UNSUPPORTED beyond). The caches, M, z, out and the workspace
 * may not overlap each other or the inputs. Checks, ownership and
 * asynchrony as for the forward.
 */
infini_status_t infini_attn_decode_workspace_size(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype, size_t* bytes);

infini_status_t infini_attn_decode_step(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t seg_len, int64_t pos,
    int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    void* k_cache, void* v_cache, float* M, float* z, void* out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The decode step with a key width different from the value width (the
 * memory M is d_key x d_value, "Infini-Attention" (AI Wiki), "How does the
 * compressive memory work?"): q [B][Hq][d_key], k [B][Hkv][d_key],
 * v [B][Hkv][d_value], k_cache [B][Hkv][seg_len][d_key], v_cache
 * [B][Hkv][seg_len][d_value], M [B][Hkv][d_key][d_value], z [B][Hkv][d_key],
 * out [B][Hq][d_value]; the scale is 1/sqrt(d_key). The fold of a complete
 * segment runs the segment-by-segment scan when d_key != d_value. Widths,
 * sizes, overlaps and errors as infini_attn_decode_step; workspace from
 * infini_attn_decode_workspace_size_kv. Identical to infini_attn_decode_step
 * when d_key == d_value.
 */
infini_status_t infini_attn_decode_workspace_size_kv(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t d_key, int64_t d_value, int64_t seg_len,
    int32_t rule, int32_t dtype, size_t* bytes);
infini_status_t infini_attn_decode_step_kv(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t d_key, int64_t d_value, int64_t seg_len,
    int64_t pos, int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    void* k_cache, void* v_cache, float* M, float* z, void* out,
    void* workspace, size_t workspace_bytes, void* stream);

/* A static, human-readable name of a status code. Never NULL. */
/*
 * Training forward: infini_attn_forward, plus the softmax statistics the
 * backward pass needs.
 *   lse: [B][Hq][L] float, written: for query row t of its segment,
 *        lse[t] = log2( sum over visible keys u of exp2(c q_t . k_u) ),
 *        c = log2(e) / sqrt(d), i.e. the base-2 log of the softmax
 *        denominator of the scaled scores, as the kernel computed it.
 * Same workspace, sizes and errors as infini_attn_forward; lse must be
 * non-NULL, 16-byte aligned and overlap no other argument.
 */
infini_status_t infini_attn_forward_train(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    void* out, float* M_final, float* z_final, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/* infini_attn_forward_train with a key width different from the value width
 * (the sizes and layouts of infini_attn_forward_kv, lse as above). */
infini_status_t infini_attn_forward_train_kv(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d_key, int64_t d_value,
    int64_t seg_len, int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    void* out, float* M_final, float* z_final, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass ("Infini-Attention" (AI Wiki), "How is an Infini-attention
 * model trained?": gradients flow through the memory recurrence from segment
 * to segment, as in truncated backpropagation through time). One call is the
 * truncation window: for the loss
 *   sum(d_out * out) + sum(dM_final * M_final) + sum(dz_final * z_final)
 * of the forward with the same arguments, it writes the gradients with
 * respect to every input, through all segments down to (M0, z0).
 *   q, k, v, beta, M0, z0: the forward's inputs;
 *   out, lse: the forward's outputs (infini_attn_forward_train);
 *   d_out: [B][Hq][L][d] element type, the gradient of out;
 *   dM_final [B][Hkv][d][d], dz_final [B][Hkv][d]: float gradients of the
 *     final state, or NULL for zero;
 *   dq, dk, dv: like q, k, v (element type), written;
 *   dbeta: [Hq] float, written (summed over the batch and the stream);
 *   dM0, dz0: like M0, z0 (float), written;
 *   workspace, workspace_bytes: at least infini_attn_backward_workspace_size
 *     (one window: the whole call).
 * Sizes and errors as infini_attn_forward. The outputs and the workspace may
 * overlap no argument. Gradients are accumulated in float and rounded to the
 * element type once, at the end.
 */
infini_status_t infini_attn_backward_workspace_size(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype, size_t* bytes);
infini_status_t infini_attn_backward(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t seg_len,
    int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    const void* out, const float* lse, const void* d_out,
    const float* dM_final, const float* dz_final,
    void* dq, void* dk, void* dv, float* dbeta, float* dM0, float* dz0,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward with a key width different from the value width ("Infini-
 * Attention" (AI Wiki), "How does the compressive memory work?": M maps
 * d_key-dimensional keys to d_value-dimensional values), for the forward of
 * infini_attn_forward_kv trained with the same loss. q, k, dq, dk are
 * [.][L][d_key]; v, dv, out, d_out [.][L][d_value]; M0, dM_final, dM0
 * [B][Hkv][d_key][d_value]; z0, dz_final, dz0 [B][Hkv][d_key]; lse from
 * infini_attn_forward_train_kv.
 * d_key, d_value in {32, 64, 128}; the rest as infini_attn_backward, which
 * these calls equal when d_key == d_value. Two widths run the product path
 * (float accumulation, one wave per row for the local attention): correct at
 * every width pair, not tuned.
 */
infini_status_t infini_attn_backward_workspace_size_kv(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d_key, int64_t d_value,
    int64_t seg_len, int32_t rule, int32_t dtype, size_t* bytes);
infini_status_t infini_attn_backward_kv(
    int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d_key, int64_t d_value,
    int64_t seg_len, int32_t rule, int32_t dtype,
    const void* q, const void* k, const void* v, const float* beta,
    const float* M0, const float* z0,
    const void* out, const float* lse, const void* d_out,
    const float* dM_final, const float* dz_final,
    void* dq, void* dk, void* dv, float* dbeta, float* dM0, float* dz0,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The block with its projections ("Infini-Attention" (AI Wiki), "What happens
 * inside the Infini-attention block?": the layer forms the usual query, key
 * and value projections of its input tokens, runs both attention paths on
 * them, and sends the gated result through the output matrix). Readings of
 * what the page leaves open: no biases; weights are stored as a linear layer
 * stores them, (out_features, in_features), and applied as x W^T; w_qkv
 * stacks the Hq query heads' d rows each, then the Hkv key heads', then the
 * Hkv value heads'; the output projection reads the heads' gated results
 * concatenated in head order (feature h d + j is element j of head h).
 *
 *   q, k, v            = the heads of x w_qkv^T
 *   a, M_final, z_final = infini_attn_forward(q, k, v, beta, M0, z0, ...)
 *   y                  = concat_h(a_h) w_o^T
 *
 * Layouts (row-major, contiguous, device memory):
 *   x, y       [B][L][d_model]         bf16
 *   w_qkv      [(Hq + 2 Hkv) d][d_model] bf16
 *   w_o        [d_model][Hq d]         bf16
 *   beta, M0, z0, M_final, z_final     as in infini_attn_forward.
 * q, k, v and a are kept in the workspace in bf16 (each rounded once, the
 * products accumulating in float), head-major as infini_attn_forward takes
 * them; the output projection reads a in place. The workspace begins with q,
 * k, v and a, in that order, each region rounded up to a multiple of 256
 * bytes (so a caller may read the projections back after the call).
 *
 * Sizes and errors: dtype must be INFINI_BF16 and d_model a multiple of 32
 * (else INFINI_ERR_UNSUPPORTED); B L < 2^31 and d_model < 2^22 (else
 * INFINI_ERR_INVALID_ARG); the rest as infini_attn_forward. The workspace must
 * hold infini_attn_block_workspace_size bytes (one window: the whole call).
 * y and the workspace overlap no argument; M_final may be M0 and z_final may
 * be z0. Asynchronous on `stream`.
 *
 * infini_attn_block_forward_timed is the same call; events[0..3], those of
 * them passed (n_events <= 4 are used), are recorded on `stream` before the
 * input projection, after it, after the block and after the output
 * projection.
 */
infini_status_t infini_attn_block_workspace_size(
    int64_t B, int64_t L, int64_t d_model, int64_t Hq, int64_t Hkv, int64_t d,
    int64_t seg_len, int32_t rule, int32_t dtype, size_t* bytes);
infini_status_t infini_attn_block_forward(
    int64_t B, int64_t L, int64_t d_model, int64_t Hq, int64_t Hkv, int64_t d,
    int64_t seg_len, int32_t rule, int32_t dtype,
    const void* x, const void* w_qkv, const void* w_o, const float* beta,
    const float* M0, const float* z0,
    void* y, float* M_final, float* z_final,
    void* workspace, size_t workspace_bytes, void* stream);
infini_status_t infini_attn_block_forward_timed(
    int64_t B, int64_t L, int64_t d_model, int64_t Hq, int64_t Hkv, int64_t d,
    int64_t seg_len, int32_t rule, int32_t dtype,
    const void* x, const void* w_qkv, const void* w_o, const float* beta,
    const float* M0, const float* z0,
    void* y, float* M_final, float* z_final,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events);

/*
 * The block with a key width different from the value width ("Infini-
 * Attention" (AI Wiki), "How does the compressive memory work?": the memory
 * maps d_key-dimensional keys to d_value-dimensional values). Query and key
 * heads are d_key wide, value heads and the gated result d_value wide:
 *   w_qkv      [(Hq + Hkv) d_key + Hkv d_value][d_model] bf16 (the Hq query
 *              heads' d_key rows each, the Hkv key heads' d_key rows, the Hkv
 *              value heads' d_value rows)
 *   w_o        [d_model][Hq d_value] bf16 (feature h d_value + j is element j
 *              of head h)
 *   M0, M_final [B][Hkv][d_key][d_value] float; z0, z_final [B][Hkv][d_key].
 * The workspace holds q [B][Hq][L][d_key], k [B][Hkv][L][d_key],
 * v [B][Hkv][L][d_value] and a [B][Hq][L][d_value] in bf16 first, in that order,
 * each rounded up to 256 bytes, then the forward's. d_key and d_value in
 * {32, 64, 128}; everything else as infini_attn_block_forward, which these
 * calls equal when d_key == d_value.
 */
infini_status_t infini_attn_block_workspace_size_kv(
    int64_t B, int64_t L, int64_t d_model, int64_t Hq, int64_t Hkv, int64_t d_key,
    int64_t d_value, int64_t seg_len, int32_t rule, int32_t dtype, size_t* bytes);
infini_status_t infini_attn_block_forward_kv(
    int64_t B, int64_t L, int64_t d_model, int64_t Hq, int64_t Hkv, int64_t d_key,
    int64_t d_value, int64_t seg_len, int32_t rule, int32_t dtype,
    const void* x, const void* w_qkv, const void* w_o, const float* beta,
    const float* M0, const float* z0,
    void* y, float* M_final, float* z_final,
    void* workspace, size_t workspace_bytes, void* stream);

/* A static, human-readable name of a status code ("unknown status" for any
 * other value). infini_attn_error_string is the same function under a second
 * name. */
const char* infini_attn_status_string(int32_t status);
const char* infini_attn_error_string(int32_t status);

/* The ABI version: major * 10000 + minor * 100 + patch. */
int32_t infini_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* INFINI_ATTN_H */
