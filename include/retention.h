/*
 * retention.h -- C ABI of libretention, the MI355X (gfx950) library for
 * chunkwise causal retention, its recurrent decode step and causal linear
 * attention with the elu+1 feature map.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major, last index fastest:
 *      q, k      [B][H][T][dk]        v, out    [B][H][T][dv]
 *      state     [B][H][dk][dv]       (rows index key features, columns value
 *                                      dimensions; always fp32)
 *    Device pointers must be 16-byte aligned.
 *  - dtype is RET_F32 or RET_BF16 and applies to q, k, v and out.  Products
 *    accumulate in fp32 and the state is fp32; out is rounded once, to
 *    nearest even, on store.
 *  - gamma is a HOST array of H floats, read during the call; each value must
 *    lie in (0, 1].  gamma = 1 is plain (unnormalised) causal linear
 *    attention with the identity feature map.
 *  - stream is a hipStream_t (passed as void*); NULL means the default
 *    stream.  Calls are asynchronous: they enqueue kernels on the stream and
 *    return.  Results are visible after the stream is synchronised.
 *  - Ownership: the caller allocates and owns every buffer, workspace
 *    included; the library allocates no device memory and keeps no pointer
 *    after the call returns.  The bf16 forward paths (retention_fwd,
 *    linear_attn_fwd) split each sequence into segments and need a device
 *    workspace for the partial segment states: ask
 *    retention_fwd_workspace_bytes / linear_attn_workspace_bytes for its size
 *    (0 when none is needed), pass a 16-byte aligned buffer of at least that
 *    many bytes that overlaps no tensor of the call.  Its contents on entry
 *    are irrelevant; calls that share a workspace must not overlap in time
 *    (the same stream, or synchronised streams).
 *  - Errors: the return value is RET_OK (0) or a negative RET_ERR_* code.
 *    Argument errors are detected on the host before anything is enqueued, so
 *    a failed call has no effect.  RET_ERR_HIP reports a failed launch.  A
 *    human-readable message for the last error of the calling thread is
 *    returned by retention_last_error().  Inputs are never modified (except
 *    the state of the two decode steps, which is updated in place).
 *  - The execution plan of a call (which kernels, how many segments, slice
 *    widths, internal chunk) is a function of its arguments only, unless the
 *    calling thread has set a plan override (retention_set_plan_override),
 *    a hook for tests and tuning.  No environment variable is read.
 *
 * Sources (page title, then passage):
 *   "RetNet" (bembew.net): the single-head definition O = (Q K^T (.) D) V with
 *       D_nm = gamma^(n-m) for n >= m; "Recurrent Representation"
 *       (S_n = gamma S_{n-1} + K_n^T V_n, O_n = Q_n S_n); "Chunked Recurrent
 *       Representation"; "Multi-Scale Retention" (one gamma per head).
 *   "Efficient and Sparse Transformers" (temporalbook 12.5), section 6: the
 *       parallel, recurrent and chunkwise forms; gamma = 1 as linear attention.
 *   "Linear attention" (zerotofrontier 21.2): box "Causal linear attention,
 *       recurrent form" (S, z, eps); the coding exercise "Causal linear
 *       attention, recurrent and parallel, plus the decode step" (one decode
 *       step on (S, z)); section "Decoding, training, and what each costs"
 *       (prefill, then decode from the prefill's state).
 */
#ifndef RETENTION_H
#define RETENTION_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RET_ABI_VERSION 11

/* element types of q, k, v, out */
#define RET_F32 0
#define RET_BF16 1

/* output normalisations for retention_fwd_normalized */
#define RET_NORM_ROWSUM 1 /* divide each row by its score row sum, floored at 1 in size */
#define RET_NORM_GROUP 2  /* then GroupNorm over the row's dv features */

/* feature maps for linear_attn_fwd */
#define RET_PHI_ELU1 1 /* phi(x) = x + 1 for x > 0, e^x otherwise */

/* return codes */
#define RET_OK 0
#define RET_ERR_NULL (-1)      /* a required pointer is NULL */
#define RET_ERR_SHAPE (-2)     /* unsupported or inconsistent sizes */
#define RET_ERR_DTYPE (-3)     /* unknown dtype */
#define RET_ERR_CHUNK (-4)     /* unsupported chunk length */
#define RET_ERR_GAMMA (-5)     /* a decay value outside (0, 1] or not finite */
#define RET_ERR_PHI (-6)       /* unknown feature map */
#define RET_ERR_ALIGN (-7)     /* a device pointer is not 16-byte aligned */
#define RET_ERR_ALIAS (-8)     /* an output overlaps an input or another output */
#define RET_ERR_WORKSPACE (-9) /* workspace NULL or smaller than the call needs */
#define RET_ERR_HIP (-10)      /* a kernel launch failed */

/*
 * retention_fwd -- causal retention over whole sequences, chunkwise form,
 * from a zero initial state.
 *
 *   out[b,h,t,:] = sum_{s<=t} gamma[h]^(t-s) (q[b,h,t,:] . k[b,h,s,:]) v[b,h,s,:]
 *
 * ("RetNet", single-head definition and "Chunked Recurrent Representation";
 * "Efficient and Sparse Transformers", section 6, "Chunkwise form".)  Inside a
 * chunk of `chunk` tokens the masked, decayed Q K^T V is computed in parallel;
 * across chunks a fp32 dk x dv state per (b, h) is carried with
 * S <- gamma^c S + (K (.) zeta)^T V.  bf16 inputs split each sequence into
 * segments whose entering states are decayed sums of the earlier segments'
 * contributions (the recurrence is linear); fp32 inputs walk whole sequences.
 * The result does not depend on `chunk` or on the split beyond rounding.
 *
 *   q, k, v      device, [B][H][T][dk|dv], dtype
 *   gamma        host, H floats in (0, 1]
 *   chunk        64 or 128
 *   out          device, [B][H][T][dv], dtype (written)
 *   final_state  device, [B][H][dk][dv] fp32, the state after token T-1
 *                (written); may be NULL.  T = 0 writes zeros.
 *   dk, dv       each 64 or 128; dv must be a multiple of 16
 *   T            >= 0, any value (a short last chunk is handled exactly)
 *   workspace    device scratch of ws_bytes bytes (see Ownership); may be
 *                NULL when retention_fwd_workspace_bytes returns 0
 */
int retention_fwd(const void *q, const void *k, const void *v, const float *gamma,
                  int chunk, void *out, float *final_state, int B, int H, int T,
                  int dk, int dv, int dtype, void *workspace, size_t ws_bytes,
                  void *stream);

/* Workspace bytes retention_fwd needs for these arguments (0: none, or the
 * arguments are invalid and the call will say why).  Host only.  The same
 * size serves retention_fwd_from_state. */
size_t retention_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                     int dtype);

/*
 * retention_fwd_noalloc -- retention_fwd for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, hosts that forbid allocation.  Same arguments and results as
 * retention_fwd (bit for bit: the same kernels and plan), without `workspace`
 * and `ws_bytes`.  The partial segment states live in a device array of the
 * library instead, RET_NOALLOC_MAX_WORKSPACE bytes on each GPU it runs on,
 * held from the first call on that GPU until the process ends.  The call
 * allocates nothing (no hipMalloc, no library allocation).
 *
 *   - Sizes whose segment states need more than RET_NOALLOC_MAX_WORKSPACE
 *     bytes (retention_fwd_workspace_bytes(...) tells) return
 *     RET_ERR_WORKSPACE; use retention_fwd with a workspace for those.  The
 *     [1, 32, 65536, 128] bf16 forward needs 14.7 MB.
 *   - Every call on one GPU shares the array: calls that overlap in time on
 *     one GPU (several streams, several host threads) race and give wrong
 *     outputs.  Calls ordered on one stream are safe.  Its contents between
 *     calls do not matter (each call writes the states before reading them).
 *   - The device is the one that runs `stream` (the current device for NULL).
 *     Its first call on a device looks up the array's address there
 *     (RET_ERR_HIP if that fails).
 */
#define RET_NOALLOC_MAX_WORKSPACE 33554432 /* bytes of segment states per GPU (32 MiB) */
int retention_fwd_noalloc(const void *q, const void *k, const void *v, const float *gamma, int chunk,
                          void *out, float *final_state, int B, int H, int T, int dk, int dv,
                          int dtype, void *stream);

/*
 * retention_fwd_from_state -- retention_fwd continued from a given state S0
 * (the state after earlier tokens, e.g. a previous call's final_state):
 *
 *   out[b,h,t,:] = gamma^(t+1) q_t S0 + sum_{s<=t} gamma^(t-s) (q_t . k_s) v_s
 *   final_state  = gamma^T S0 + sum_s gamma^(T-1-s) k_s v_s^T
 *
 * i.e. the recurrence of "RetNet", "Recurrent Representation", started from S0
 * instead of zero; running a sequence in pieces, each from the previous
 * piece's final state, gives the result of one call over the whole sequence.
 *
 *   initial_state  device, [B][H][dk][dv] fp32, read only; may be NULL (zero).
 *                  It may alias q, k or v but not out or final_state.
 *   other arguments as retention_fwd; T = 0 copies initial_state to
 *   final_state.
 */
int retention_fwd_from_state(const void *q, const void *k, const void *v,
                             const float *gamma, int chunk, const float *initial_state,
                             void *out, float *final_state, int B, int H, int T, int dk,
                             int dv, int dtype, void *workspace, size_t ws_bytes,
                             void *stream);

/*
 * retention_fwd_normalized -- retention_fwd (zero initial state) with the
 * output normalisation of a RetNet layer fused into the chunk walk:
 *
 *   n_t   = gamma n_{t-1} + k_t             (decayed key sum, dk)
 *   out_t = (q_t S_t) / max(|n_t . q_t|, 1)
 *
 * n_t . q_t is the row sum of the decayed scores, sum_{s<=t} gamma^(t-s)
 * q_t . k_s ("Linear attention", box "An LSTM whose cell is linear
 * attention", with forget gate gamma and input gate 1, and the remark that
 * RetNet divides each score row by the absolute value of its sum clamped
 * below at 1).  RET_NORM_GROUP then replaces each row by
 * (out - mean(out)) / sqrt(var(out) + eps), population variance over the
 * head's dv features, no learned gain or bias ("RetNet", the layer's
 * optional GroupNorm).  Statistics are taken in fp32 before the single
 * rounding to the output dtype.
 *
 *   dtype    RET_BF16 (segment walk) or RET_F32 (value-slice walk).  fp32
 *            GroupNorm is fused into the walk where one workgroup holds whole
 *            output rows (chunk 64 with dv = 64 or dk = 64, dv = 128; chunk
 *            128 with dk = dv = 64); elsewhere the walk applies the floor and
 *            a second pass over `out` standardises each row in place
 *   norm     RET_NORM_ROWSUM or RET_NORM_GROUP (RET_ERR_SHAPE otherwise)
 *   eps      GroupNorm epsilon, finite and > 0 (1e-5 is usual); a row whose
 *            values are all equal (zero queries) then comes out as zeros.
 *            Ignored by RET_NORM_ROWSUM (any finite value >= 0)
 *   workspace  retention_fwd_normalized_workspace_bytes(...) bytes
 *   chunk    64 or 128; bf16 with dk = dv = 128 walks 64 (LDS), same result
 *   other arguments as retention_fwd (no final state)
 */
int retention_fwd_normalized(const void *q, const void *k, const void *v, const float *gamma,
                             int chunk, int norm, float eps, void *out, int B, int H, int T,
                             int dk, int dv, int dtype, void *workspace, size_t ws_bytes,
                             void *stream);

/* Workspace bytes retention_fwd_normalized needs (0: none or invalid).  Host only. */
size_t retention_fwd_normalized_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                                int dtype);

/*
 * retention_bwd -- gradients of retention_fwd (zero initial state) with
 * respect to q, k and v, given dout = dL/dout for a scalar loss L:
 *
 *   dq_t = S_t dout_t,          S_t = sum_{s<=t} gamma^(t-s) k_s v_s^T
 *   dk_s = U_s v_s,  dv_s = U_s^T k_s,   U_s = sum_{t>=s} gamma^(t-s) q_t dout_t^T
 *
 * ("Linear attention", section "Decoding, training, and what each costs": the
 * gradients of the causal recurrence are cumulative sums too, forward in time
 * for the queries and backward in time for the keys and values; "RetNet",
 * single-head definition, for the operator being differentiated.)  Computed
 * as three chunkwise walks: dq is the forward of (dout, v, k), dk and dv are
 * forwards of (v, dout, q) and (k, q, dout) over the time-reversed sequence.
 *
 *   q, k, v, dout  device, [B][H][T][dk|dv], dtype, read only
 *   dq, dk, dv     device, [B][H][T][dk|dk|dv], dtype (written); none may
 *                  overlap an input or another gradient
 *   gamma, chunk, B, H, T, dk, dv, dtype: as retention_fwd
 *   workspace      device scratch of retention_bwd_workspace_bytes(...) bytes
 */
int retention_bwd(const void *q, const void *k, const void *v, const float *gamma, int chunk,
                  const void *dout, void *dq, void *dk, void *dv, int B, int H, int T,
                  int d_k, int d_v, int dtype, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes retention_bwd needs for these arguments (0: none, or the
 * arguments are invalid).  Host only. */
size_t retention_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype);

/*
 * retention_bwd_from_fwd -- retention_bwd for a training step whose forward
 * kept its workspace.  The query gradient dq_t = S_t dout_t walks the forward
 * recurrence S_t = gamma S_{t-1} + v_t k_t^T with the roles of keys and values
 * swapped; its per-segment state sums are the transposes of the ones the
 * forward (S_t = gamma S_{t-1} + k_t v_t^T, "RetNet", recurrent
 * representation) left in its workspace.  Reading those instead of summing
 * them again saves one read of k and v over all but the last segment.
 *
 *   fwd_workspace  device, read only: the workspace of a retention_fwd or
 *                  retention_fwd_from_state call that completed earlier in
 *                  stream order, with the same k, v, gamma, chunk, B, H, T,
 *                  dk, dv and dtype (the initial state does not matter), not
 *                  written since; it may be NULL when that call needed none
 *                  (retention_fwd_workspace_bytes(...) == 0).  The library
 *                  cannot check that it holds those states: a different
 *                  buffer gives wrong dq without an error.
 *   fwd_ws_bytes   its size; at least retention_fwd_workspace_bytes(...)
 *   everything else: as retention_bwd, including `workspace`, which must be a
 *                  separate buffer of retention_bwd_workspace_bytes(...) bytes
 *
 * Errors: those of retention_bwd; RET_ERR_WORKSPACE when fwd_workspace is
 * NULL or short although the forward needed one; RET_ERR_ALIGN when it is not
 * 16-byte aligned; RET_ERR_ALIAS when it overlaps dq, dk, dv or `workspace`.
 * If a plan override changed the forward's segment plan between the calls,
 * dq runs its own state pass (the result is unchanged).
 */
int retention_bwd_from_fwd(const void *q, const void *k, const void *v, const float *gamma, int chunk,
                           const void *dout, const void *fwd_workspace, size_t fwd_ws_bytes, void *dq,
                           void *dk, void *dv, int B, int H, int T, int d_k, int d_v, int dtype,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * retention_decode_step -- one recurrent step for N sequences x H heads,
 * updating state in place, then reading the output from the updated state:
 *
 *   S <- gamma[h] S + k v^T,   out = q S
 *
 * ("RetNet", "Recurrent Representation"; "Efficient and Sparse
 * Transformers", section 6, recurrent form and its minimal recurrent step.)
 *
 *   q, k    device, [N][H][dk], dtype       v, out  device, [N][H][dv], dtype
 *   state   device, [N][H][dk][dv] fp32, read and written in place
 *   gamma   host, H floats in (0, 1]
 *   dk, dv  each 64 or 128
 */
int retention_decode_step(const void *q, const void *k, const void *v,
                          const float *gamma, float *state, void *out, int N, int H,
                          int dk, int dv, int dtype, void *stream);

/*
 * linear_attn_fwd -- causal linear attention with a positive feature map and
 * its normaliser, chunkwise (internal chunk 128; 64 for bf16 with dk = 128):
 *
 *   S_t = S_{t-1} + phi(k_t) v_t^T,  z_t = z_{t-1} + phi(k_t),
 *   out_t = S_t^T phi(q_t) / (z_t^T phi(q_t) + eps)
 *
 * ("Linear attention", box "Causal linear attention, recurrent form", and
 * theorem "Recurrent and parallel forms agree".)  Zero initial S and z.
 *
 *   q, k, v    device, [B][H][T][dk|dv], dtype     out  device, [B][H][T][dv]
 *   phi        RET_PHI_ELU1
 *   eps        >= 0 (the pages use 1e-6)
 *   dk, dv     each 64 or 128; T >= 0
 *   workspace  device scratch of ws_bytes bytes (see Ownership); may be NULL
 *              when linear_attn_workspace_bytes returns 0
 */
int linear_attn_fwd(const void *q, const void *k, const void *v, int phi, void *out,
                    int B, int H, int T, int dk, int dv, int dtype, float eps,
                    void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes linear_attn_fwd needs for these arguments (0: none, or the
 * arguments are invalid).  Host only.  The same size serves
 * linear_attn_fwd_from_state. */
size_t linear_attn_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype);

/*
 * linear_attn_fwd_from_state -- linear_attn_fwd started from (S0, z0), the
 * state and normaliser after earlier tokens, and optionally returning the pair
 * after the last token, so a prefill can hand its (S, z) to
 * linear_attn_decode_step ("Linear attention", the decode-step exercise and
 * section "Decoding, training, and what each costs").
 *
 *   initial_S  device, [B][H][dk][dv] fp32, read only; NULL means zero
 *   initial_z  device, [B][H][dk] fp32, read only; NULL means zero
 *   final_S    device, [B][H][dk][dv] fp32 (written); may be NULL
 *   final_z    device, [B][H][dk] fp32 (written); may be NULL
 *   The initial pair may alias q, k or v; no output may overlap an input or
 *   another output.  Other arguments as linear_attn_fwd; T = 0 copies the
 *   initial pair to the final one.
 */
int linear_attn_fwd_from_state(const void *q, const void *k, const void *v, int phi,
                               const float *initial_S, const float *initial_z, void *out,
                               float *final_S, float *final_z, int B, int H, int T,
                               int dk, int dv, int dtype, float eps, void *workspace,
                               size_t ws_bytes, void *stream);

/*
 * linear_attn_decode_step -- one decode step of causal linear attention for
 * N sequences x H heads, updating (S, z) in place, then reading the output
 * from the updated pair:
 *
 *   S <- S + phi(k) v^T,  z <- z + phi(k),  out = S^T phi(q) / (z^T phi(q) + eps)
 *
 * ("Linear attention", the coding exercise "Causal linear attention, recurrent
 * and parallel, plus the decode step": the token is included in its own sum.
 * The exercise returns new arrays; this call works in place, like
 * retention_decode_step, and a caller that needs the old pair copies it.)
 *
 *   q, k    device, [N][H][dk], dtype       v, out  device, [N][H][dv], dtype
 *   S       device, [N][H][dk][dv] fp32, read and written in place
 *   z       device, [N][H][dk] fp32, read and written in place
 *   phi     RET_PHI_ELU1;  eps >= 0 (the pages use 1e-6);  dk, dv each 64 or 128
 */
int linear_attn_decode_step(const void *q, const void *k, const void *v, int phi,
                            float *S, float *z, void *out, int N, int H, int dk, int dv,
                            int dtype, float eps, void *stream);

/*
 * gla_fwd -- causal gated linear attention with one data-dependent gate per
 * token and key channel, chunkwise (64-token chunks), from a zero state:
 *
 *   S_t[c][n] = exp(lg_t[c]) S_{t-1}[c][n] + k_t[c] v_t[n],   out_t = q_t S_t
 *
 * ("Efficient and Sparse Transformers", section "Gated Linear Attention:
 * Toward Input-Dependent Forgetting": RetNet's fixed decay becomes a learned
 * gate applied element-wise to the state; here the gate of key channel c,
 * shared by the value columns.  lg = log(gamma) for every channel is
 * retention, lg = 0 plain linear attention.)  Inside a chunk the gates are
 * folded into the operands, each scaled by exponentials of log-gate sums
 * relative to its 16-token tile (every folded operand at most its raw
 * magnitude); a chunk holding a 16-token tile whose gate sum falls below -80
 * in some channel forms its scores term by term with exponents
 * e^{b_i - b_j} <= 1.
 *
 *   q, k            device, [B][H][T][dk], dtype
 *   log_gate        device, [B][H][T][dk] fp32 whatever the dtype; finite
 *                   and <= 0 (a value above 0, a gate above 1, is taken as
 *                   0; NaN propagates; accuracy assumes |log_gate| of order
 *                   1-10 per token; -inf is not accepted by the chunk form)
 *   v, out          device, [B][H][T][dv], dtype
 *   final_state     device, [B][H][dk][dv] fp32 (written); may be NULL
 *   dtype           RET_F32 or RET_BF16 (q, k, v, out); fp32 arithmetic
 *   dk, dv          each 64 or 128
 *   workspace       gla_fwd_workspace_bytes(...) bytes: per segment but the
 *                   last, its state contribution and per-channel gate totals
 */
int gla_fwd(const void *q, const void *k, const void *v, const float *log_gate, void *out,
            float *final_state, int B, int H, int T, int dk, int dv, int dtype,
            void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes gla_fwd needs (0: none or invalid).  Host only. */
size_t gla_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype);

/* forward paths for retention_set_plan_override */
#define RET_PATH_AUTO 0    /* the library's choice */
#define RET_PATH_SLICE 1   /* value-slice walk (fp32's path; bf16 only when forced) */
#define RET_PATH_SEGMENT 2 /* segment-split walk where the dtype has one (bf16) */

/*
 * retention_set_plan_override -- testing and tuning hook.  Fixes parts of the
 * plan that every later call made from the CALLING HOST THREAD would
 * otherwise choose from its arguments, until the next call of this function;
 * other threads are unaffected.  retention_set_plan_override(0, 0, 0, 0)
 * restores the automatic plan.  No override changes results beyond floating-
 * point rounding order; an override a kernel cannot honour (a slice width
 * whose variant does not fit, the segment path for fp32) is ignored.
 *
 *   fwd_path   RET_PATH_AUTO, RET_PATH_SLICE or RET_PATH_SEGMENT
 *   segments   0 (automatic) or the segment count per (b, h) sequence
 *              (capped at the number of chunks), for every chunked walk
 *   walk_nt    0 (automatic) or a narrower value slice of the slice path, in
 *              16-column tiles: 1, 2, 4 or 8
 *   lin_chunk  0 (automatic), 64 or 128: the chunk of bf16 linear attention
 *              on the segment path (128 needs dk = 64)
 *
 * The workspace-size helpers follow the same override, so a workspace sized
 * under one override must be used under the same override.  Returns RET_OK,
 * or RET_ERR_SHAPE / RET_ERR_CHUNK for an out-of-range value (the previous
 * override then stays in place).  Host only; enqueues nothing.
 */
int retention_set_plan_override(int fwd_path, int segments, int walk_nt, int lin_chunk);

/* Message describing the last error returned on the calling thread ("" if
 * none).  The pointer stays valid until the next call on that thread. */
const char *retention_last_error(void);

/* RET_ABI_VERSION of the loaded library. */
int retention_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RETENTION_H */
