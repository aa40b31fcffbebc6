/*
 * jagged_attn.h — C ABI of the MI355X (gfx950) jagged attention library.
 *
 * Two attention forms over jagged (variable-length, unpadded) batches, with
 * forward and backward passes:
 *
 *   GDPA (generalized dot-product attention):
 *       O_i = sum_{valid j} act(scale * <q_i, k_j> + bias_ij) v_j
 *     act is SiLU or GELU and there is no row normalisation.  The pages
 *     describe the attention-like modules as two matrix products with an
 *     element-wise activation in between, GELU or SiLU replacing softmax
 *     ("GEM Training: How Meta Doubled the Efficiency...", section
 *     "What to watch"; "Meta redesigns AI training infrastructure...", section
 *     "Custom Kernels and 5D Parallelism for Trillion-Parameter Scale").
 *
 *   JFA (jagged flash attention):
 *       O_i = sum_{valid j} softmax_j(scale * <q_i, k_j> + bias_ij) v_j
 *     FlashAttention run directly on jagged tensors with custom attention
 *     biases, asymmetric query / key-value lengths and a backward pass
 *     ("GEM Training...", section "What happened"; "Meta redesigns...",
 *     section "Eliminating Compute Waste in Asymmetric Workloads").
 *
 * Data layout.  Values are token-major [T, H, D], contiguous (row stride H*D
 * elements), bf16 or fp32.  Sample b owns query rows q_offsets[b] ..
 * q_offsets[b+1]-1 and key / value rows kv_offsets[b] .. kv_offsets[b+1]-1;
 * offsets are int32 [B+1], start at 0, never decrease and end at the row
 * count.  Samples may be empty.  Within a sample, i and j are 0-based local
 * positions and a pair (i, j) is valid iff j < Lk and, with causal masking,
 * j <= i + Lk - Lq (bottom-right alignment; j <= i when Lq == Lk).  A sliding
 * window w > 0 (window) also requires ia - j < w and, without causal masking,
 * j - ia < w, where ia = i + Lk - Lq is the row's aligned position: each row
 * sees the w nearest keys up to its diagonal (causal) or a band of 2w - 1
 * keys around it.  The pages name sliding-window attention ("Meta redesigns
 * AI training infrastructure...", section "Custom Kernels and 5D Parallelism
 * for Trillion-Parameter Scale") without defining it; this is the plain
 * reading.
 *
 * Shared query block.  With q_offsets == NULL, q holds lq_fixed rows
 * ([lq_fixed, H, D]) that every sample attends with (pooling by learned seed
 * queries); the output still has one row block per sample:
 * [B * lq_fixed, H, D], sample b at rows b * lq_fixed.  Forward only.
 *
 * Rotary embedding.  With rope_base > 0 every query and key row is turned
 * before the scores are formed: element d < D/2 and element d + D/2 of a row at
 * sample-local position t (query i, key j; row r of a shared query block) turn
 * by the angle t * rope_base^(-2d/D):
 *   x'_d = x_d cos a - x_{d+D/2} sin a,   x'_{d+D/2} = x_d sin a + x_{d+D/2} cos a
 * (RoFormer's rotation in split-half form; values are not turned).  The pages
 * name a rotary embedding fused into their block-attention kernel ("Meta
 * redesigns AI training infrastructure...", section "Custom Kernels and 5D
 * Parallelism for Trillion-Parameter Scale") without defining it.  Each turned
 * element is the nearest bf16 (fp32 tensors: float32) value to the turn worked
 * in fp64.  Either the call turns q and k into workspace copies, or the caller
 * turns them once with jagged_rope and passes the turned rows to both passes
 * (rope_inputs_turned = 1).  The backward entry points return gradients with
 * respect to the rows before the turn: the bf16 backward units turn their dq
 * rows back in registers before storing them, and a streaming pass turns dk
 * back (fp32: dq and dk).
 *
 * Bias.  An fp32 table [H][bias_hi - bias_lo + 1] on the device, added after
 * the scale, before the activation / softmax:
 *   JA_BIAS_REL     table[h][clamp(i - j, bias_lo, bias_hi) - bias_lo]
 *   JA_BIAS_KEYPOS  table[h][clamp(j, bias_lo, bias_hi) - bias_lo]
 * The backward entry points can also return the table's gradient (dbias,
 * below).
 *
 * Ownership.  Every buffer belongs to the caller, including the workspace
 * (ja_workspace_size bytes, 256-byte aligned, device memory).  The library
 * allocates no device memory and keeps no state between calls besides loaded
 * code objects; it may be called from several host threads on different
 * streams with different workspaces.  Calls sharing one workspace must be
 * ordered (same stream).
 *
 * Empty tensors.  A tensor with no rows (total_q, total_k or the output rows
 * equal to 0) is never read or written, and its pointer may be NULL.
 *
 * Errors.  The return code is the only error channel.  Host-visible arguments
 * are checked before anything is launched; on any error nothing is launched
 * and no output is touched.  Offsets live in device memory and are not read by
 * the host: offsets that break the rules above (including a max_kv_len bound
 * that some sample exceeds) give undefined results -- unless the environment
 * variable JA_CHECK_OFFSETS is set to 1 when the call is made.  Then, before
 * any other launch, a validation kernel checks them on the device and the call
 * waits for its verdict (it synchronises `stream`, so this mode is for
 * debugging, not for graph capture): invalid offsets return JA_ERR_BAD_OFFSETS
 * with no attention kernel launched and no output touched.  Its flag lives in
 * the workspace.  A window wider than every sample's aligned distances keeps
 * every pair: values past total_q + total_k are treated as that width.
 *
 * Asynchrony.  Every entry point enqueues its kernels on `stream` (a
 * hipStream_t, NULL for the default stream) and returns without waiting.
 * Outputs are fully overwritten (never accumulated); rows with no valid key
 * get O = 0 (JFA: LSE = -inf) and all their gradients are 0.
 */
#ifndef JAGGED_ATTN_H
#define JAGGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JA_OK = 0,
    JA_ERR_NULL = 1,        /* a required pointer is NULL */
    JA_ERR_SHAPE = 2,       /* B, H, D, total rows or bias range out of range */
    JA_ERR_UNSUPPORTED = 3, /* dtype / head_dim / act / bias kind / shared-query backward, or a
                               [rows, H, D] tensor of 4 GiB or more (split such a batch) */
    JA_ERR_WORKSPACE = 4,   /* workspace NULL, misaligned or smaller than ja_workspace_size */
    JA_ERR_BAD_OFFSETS = 5, /* offsets break the layout rules; reported only in the opt-in
                               validation mode (environment JA_CHECK_OFFSETS=1, see Errors) */
    JA_ERR_HIP = 6          /* a HIP launch failed (the HIP error is in ja_last_hip_error) */
} ja_status;

typedef enum { JA_BF16 = 0, JA_F32 = 1 } ja_dtype;
typedef enum { JA_ACT_SILU = 0, JA_ACT_GELU_TANH = 1, JA_ACT_GELU_ERF = 2 } ja_act;
typedef enum { JA_BIAS_NONE = 0, JA_BIAS_REL = 1, JA_BIAS_KEYPOS = 2 } ja_bias_kind;
typedef enum {
    JA_PASS_FWD = 0,
    JA_PASS_BWD = 1,
    JA_PASS_BWD_DBIAS = 2 /* backward that also returns the bias-table gradient */
} ja_pass;

/* Problem description: sizes by value, device pointers to the offsets and the
 * bias table.  The struct itself is read on the host during the call only. */
typedef struct ja_problem {
    int32_t batch;               /* B >= 1 samples */
    int32_t heads;               /* H >= 1 */
    int32_t head_dim;            /* D in {32, 64, 128} */
    int32_t dtype;               /* ja_dtype of q, k, v, o, dout, dq, dk, dv */
    int64_t total_q;             /* rows of q: q_offsets[B], or lq_fixed when shared */
    int64_t total_k;             /* rows of k and v: kv_offsets[B] */
    const int32_t *q_offsets;    /* device [B+1], or NULL for a shared query block */
    int32_t lq_fixed;            /* rows of the shared query block (q_offsets == NULL) */
    int32_t causal;              /* 0 or 1 */
    const int32_t *kv_offsets;   /* device [B+1] */
    float scale;                 /* multiplies <q, k> (commonly 1/sqrt(D)) */
    int32_t act;                 /* ja_act (GDPA only; ignored by JFA) */
    int32_t bias_kind;           /* ja_bias_kind */
    int32_t bias_lo, bias_hi;    /* bias index range, bias_lo <= bias_hi */
    const float *bias_table;     /* device fp32 [H][bias_hi - bias_lo + 1], or NULL when no bias */
    int32_t max_kv_len;          /* 0 = unknown, else an upper bound on every sample's key count
                                    (kv_offsets[b+1] - kv_offsets[b]).  At most 32 lets the
                                    library skip launching its long-sequence kernels; a bound
                                    that some sample exceeds gives undefined results, like
                                    invalid offsets.  Negative: JA_ERR_SHAPE. */
    int32_t window;              /* sliding window w (0 = none, negative: JA_ERR_SHAPE) */
    float rope_base;             /* rotary embedding base (commonly 10000), 0 = none; negative,
                                    infinite or NaN: JA_ERR_SHAPE */
    int32_t rope_inputs_turned;  /* with rope_base > 0: 1 = q and k are passed already turned
                                    (jagged_rope's output for this problem), so the call turns
                                    nothing on the way in and its workspace holds no turned
                                    copies; a backward still returns dq and dk for the rows
                                    before the turn.  0 = q and k as they are.  Else
                                    JA_ERR_SHAPE. */
} ja_problem;

/* Workspace bytes that the given pass of either attention form needs (0 only
 * for invalid problems).  Depends on B, H, D, total_q, total_k, lq_fixed,
 * dtype and whether the call turns q and k itself (rope_base > 0 and
 * rope_inputs_turned 0: room for the turned copies), and for
 * JA_PASS_BWD_DBIAS also on the bias range; the same value serves GDPA and
 * JFA. */
size_t ja_workspace_size(const ja_problem *p, int pass);

/* GDPA forward.  q [Tq, H, D] (or [lq_fixed, H, D]), k, v [Tk, H, D],
 * o [Tq_out, H, D] written. */
ja_status jagged_gdpa_fwd(const ja_problem *p, const void *q, const void *k, const void *v, void *o,
                          void *workspace, size_t workspace_bytes, void *stream);

/* GDPA backward of L = <O, dout>: dq [Tq, H, D], dk, dv [Tk, H, D] written.
 * Needs q_offsets (no shared query block).
 *
 * dbias (optional, NULL to skip): device fp32 [H][bias_hi - bias_lo + 1],
 * written with dL/dtable: entry c of head h sums dX_ij = dL/dX_ij over the
 * valid pairs (i, j) of every sample that read it (REL: clamp(i - j), KEYPOS:
 * clamp(j)), the bias being additive in X.  Needs a bias kind and a table
 * row of at most 4096 entries (else JA_ERR_UNSUPPORTED), and a workspace of
 * ja_workspace_size(p, JA_PASS_BWD_DBIAS) bytes (else JA_ERR_WORKSPACE); that
 * workspace holds a row of table sums per 32 query rows and head (about
 * H * (total_q / 32 + 4 B) * (bias_hi - bias_lo + 1) * 4 bytes), so the sums
 * stay deterministic bit for bit.
 * The custom biases are listed on "GEM Training: How Meta Doubled the
 * Efficiency...", section "What happened". */
ja_status jagged_gdpa_bwd(const ja_problem *p, const void *q, const void *k, const void *v,
                          const void *dout, void *dq, void *dk, void *dv, float *dbias,
                          void *workspace, size_t workspace_bytes, void *stream);

/* JFA forward.  o as for GDPA; lse fp32 [H, Tq_out] (head-major) receives the
 * natural-log row log-sum-exp of the scores, -inf for rows with no valid key.
 * o_residual (optional, NULL to skip; bf16 only, same shape as o) receives
 * fp32(O) - bf16(O), the rounding residual of the bf16 output. */
ja_status jagged_attn_fwd(const ja_problem *p, const void *q, const void *k, const void *v, void *o,
                          float *lse, void *o_residual, void *workspace, size_t workspace_bytes,
                          void *stream);

/* JFA forward that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics and outputs as
 * jagged_attn_fwd without the workspace: its plan counters and unit lists live
 * in a built-in device array of JA_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * held until the process ends (its address is looked up on the first call on
 * each device).  A problem whose forward workspace (ja_workspace_size(p,
 * JA_PASS_FWD)) exceeds it returns JA_ERR_WORKSPACE with nothing launched; with a
 * rotary embedding the turned copies of q and k count towards it.  Every call on
 * one GPU uses that GPU's array: calls that may overlap on one GPU (different
 * streams, different host threads) race on it and must be ordered by the caller.
 * The array needs no clearing: the planner kernel resets what the attention
 * kernels count from. */
#define JA_NOALLOC_SCRATCH_BYTES (4u << 20)
ja_status jagged_attn_fwd_noalloc(const ja_problem *p, const void *q, const void *k, const void *v,
                                  void *o, float *lse, void *o_residual, void *stream);

/* Rotary embedding on its own: q_turned [Tq, H, D] (or [lq_fixed, H, D]) and
 * k_turned [Tk, H, D] receive q and k turned as described under "Rotary
 * embedding" (positions from the problem's offsets), in p->dtype.  The outputs
 * may be the inputs themselves (turned in place).  Feed them to the attention
 * calls with rope_inputs_turned = 1: one turn serves a forward and its
 * backward.  Needs rope_base > 0 (else JA_ERR_SHAPE); otherwise the same
 * problem checks as a forward.  No workspace; offsets are not validated here
 * (JA_CHECK_OFFSETS applies to the attention calls).  Asynchronous on the
 * stream. */
ja_status jagged_rope(const ja_problem *p, const void *q, const void *k, void *q_turned, void *k_turned,
                      void *stream);

/* MXFP8 forward (GDPA and JFA).  The pages report MXFP8-based attention, the
 * quantisation fused into the upstream projection and normalisation kernels
 * ("Meta redesigns AI training infrastructure...", sections "Custom Kernels
 * and 5D Parallelism for Trillion-Parameter Scale" and "Key Numbers"), so q,
 * k and v arrive quantised in the OCP Microscaling MXFP8 format:
 *   q, k, v        uint8 [rows, H, D]: FP8 E4M3 codes (bias 7, no infinities,
 *                  largest finite 448);
 *   q/k/v_scale    uint8 [rows, H, D / 32]: one E8M0 scale code E per block of
 *                  32 consecutive head-dimension elements of a row and head,
 *                  scale 2^(E - 127), E in 1 .. 254 (0 and 255 are not decoded).
 * The element value is scale times code value; attention is computed exactly
 * as by jagged_gdpa_fwd / jagged_attn_fwd on those values (they are decoded to
 * bf16 exactly, accumulation in fp32).  p->dtype must be JA_BF16 (the type of
 * o and o_residual) and p->rope_base 0, else JA_ERR_UNSUPPORTED; a NULL scale
 * array of a tensor with rows: JA_ERR_NULL.  Workspace as for the forward
 * (ja_workspace_size(p, JA_PASS_FWD)).  There is no MXFP8 backward. */
ja_status jagged_gdpa_fwd_mx(const ja_problem *p, const void *q, const void *q_scale, const void *k,
                             const void *k_scale, const void *v, const void *v_scale, void *o, void *workspace,
                             size_t workspace_bytes, void *stream);
ja_status jagged_attn_fwd_mx(const ja_problem *p, const void *q, const void *q_scale, const void *k,
                             const void *k_scale, const void *v, const void *v_scale, void *o, float *lse,
                             void *o_residual, void *workspace, size_t workspace_bytes, void *stream);

/* JFA backward: takes the forward's o and lse; dq, dk, dv written.  The softmax
 * backward needs delta_i = <dO_i, O_i>.  With o_residual NULL it is formed from
 * the bf16 o alone (as FlashAttention does): o's rounding then perturbs every
 * dS_ij of a row by P_ij times that error, which dominates rows whose gradient
 * is small by cancellation.  Passing the forward's o_residual forms delta from
 * o + o_residual, exact to fp32 rounding.  Ignored for fp32 tensors.
 * dbias as for jagged_gdpa_bwd, with dX_ij = P_ij (dP_ij - delta_i). */
ja_status jagged_attn_bwd(const ja_problem *p, const void *q, const void *k, const void *v,
                          const void *o, const void *o_residual, const void *dout,
                          const float *lse, void *dq, void *dk, void *dv, float *dbias,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Measurement aid.  Kernels a call may launch: */
typedef enum {
    JA_KERNEL_PLAN = 0,       /* work-list planner */
    JA_KERNEL_FWD = 1,        /* forward attention, samples with > 32 keys */
    JA_KERNEL_BWD_FUSED = 2,  /* backward, samples with <= 32 keys */
    JA_KERNEL_BWD_KV = 3,     /* backward dK/dV units */
    JA_KERNEL_BWD_Q = 4,      /* backward dQ units */
    JA_KERNEL_BWD_DELTA = 5,  /* JFA backward delta preprocess */
    JA_KERNEL_FWD_SHORT = 6,  /* forward attention, samples with <= 32 keys */
    JA_KERNEL_BWD_DBIAS = 7,  /* bias-table gradient (both of its kernels) */
    JA_KERNEL_ROPE = 8,       /* rotary embedding of q and k (one launch) */
    JA_KERNEL_ROPE_BACK = 9,  /* backward: dq and dk turned back (one launch) */
    JA_KERNEL_CHECK_OFFSETS = 10 /* offsets validation (JA_CHECK_OFFSETS=1 only) */
} ja_kernel_id;

/* From now on, in every call made by the calling thread, record start_event
 * immediately before and stop_event immediately after launching kernel
 * `kernel_id`, on the call's stream (both are hipEvent_t created by the
 * caller).  Each kernel id has its own pair, so several kernels can be timed in
 * one call; NULL events switch that id off.  Thread-local; never synchronises. */
ja_status ja_profile_kernel(int kernel_id, void *start_event, void *stop_event);

/* Measurement aid for the work scheduler: from now on, in every call made by the
 * calling thread, each workgroup of kernel `kernel_id` (one of the persistent
 * attention kernels: JA_KERNEL_FWD, _FWD_SHORT, _BWD_KV, _BWD_Q, _BWD_FUSED, and the
 * first kernel of JA_KERNEL_BWD_DBIAS) writes
 * the shader clock cycles from its start to its exit (after its last unit) into
 * device_buffer[workgroup] (uint64, `capacity` entries; workgroups past it write
 * nothing).  Busy time max / mean over the workgroups measures the load balance.
 * The buffer stays owned by the caller and must stay valid while such calls run;
 * the library never clears it (entries past the launch's grid keep their old
 * contents).  Other kernel ids are accepted and record nothing.  NULL and 0
 * switch it off.  Errors: JA_ERR_UNSUPPORTED for an unknown id, JA_ERR_SHAPE when
 * only one of buffer and capacity is zero, or capacity < 0.  Thread-local; never
 * synchronises. */
ja_status ja_profile_busy(int kernel_id, void *device_buffer, int capacity);

/* Human-readable name of a status code (static storage). */
const char *ja_status_string(int status);

/* The HIP error code of the most recent JA_ERR_HIP in the calling thread. */
int ja_last_hip_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int ja_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JAGGED_ATTN_H */
