/*
 * linattn.h -- C ABI of liblinattn.so: chunkwise causal linear attention with
 * a constant decay per head, for AMD Instinct MI355X (gfx950).
 *
 * The method.  For every sequence (b, h) -- or every segment of it, see
 * `nseg` -- with decay lambda = lambda[h], the library computes
 *
 *     S_t = lambda * S_{t-1} + k_t v_t^T          (state, d_k x d_v, fp32)
 *     o_t = q_t^T S_t                             (output row, length d_v)
 *
 * for t = 1..L starting from the initial state S_0 and returns S_end = S_L.
 *  - The state is the per-sequence memory state, whose size does not grow
 *    with the sequence, and the evaluation is right-product-first: LASP-2
 *    (Rethinking Sequence Parallelism for Linear Attention and Its Hybrid),
 *    abstract.
 *  - Work is tiled into 64-token chunks: exact causal attention inside a
 *    chunk, the state (kernel trick) between chunks -- the split the
 *    Lightning Attention-2 entry of the LASP-2 page's related-paper list
 *    describes.
 *  - A sequence can be cut into segments that each start from a given initial
 *    state, and per-segment states combine by the scan of la_state_scan; this
 *    is what the All-Scan collective of ZeCO (Zero Communication Overhead
 *    Sequence Parallelism for Linear Attention), abstract, delivers to each
 *    rank, and what LASP-2's single all-gather of memory states feeds.
 * There is no feature map, normaliser or softmax scale: callers fold any
 * scale into q and k.  The current token is included in its own output, and
 * S_0 is decayed once before the first token is added.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (including lambda), contiguous,
 *    row-major, 16-byte aligned.  The caller owns every buffer; the library
 *    allocates and frees nothing and keeps no device state, except the fixed
 *    array of la_chunk_fwd_noalloc (below).
 *  - Token tensors: Q, K, dQ, dK are [B, H, L, dk]; V, O, dO, dV are
 *    [B, H, L, dv], all of element type `dtype`.  States (S0, S_end, dS_end,
 *    dS0) are fp32 [B, H, nseg, dk, dv] with the state row-major as [dk][dv].
 *    lambda is fp32 [H].
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *    the default stream).  The library never synchronises.  Concurrent calls
 *    on different streams are allowed if their output buffers and workspaces
 *    do not overlap.
 *  - Errors: every argument is checked on the host before any HIP call.  A
 *    check that fails returns LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED or
 *    LA_ERR_WORKSPACE, launches nothing and writes nothing.  A failed launch
 *    returns LA_ERR_HIP.  la_last_error() describes the last failure of the
 *    calling thread.  No C++ exception crosses this interface.
 *  - Preconditions that are not checked (device data is not read on the
 *    host): 0 <= lambda[h] <= 1 (lambda = 0 gives lambda^0 = 1 and every
 *    higher power 0; no entry point divides by lambda except la_decay_grad,
 *    which needs lambda[h] > 0).  Other values give undefined numbers (but no
 *    out-of-bounds access).  NaN and Inf inputs propagate.
 *  - Outputs are fully overwritten, never accumulated into.  No input may
 *    overlap an output except where stated.
 *  - Results are deterministic: the same call on the same inputs gives the
 *    same bits (no atomics).
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1,  /* null required pointer, negative size, misalignment, bad enum */
  LA_ERR_UNSUPPORTED = 2,  /* valid but not implemented: d not in {64,128}, dk != dv */
  LA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than *_workspace_bytes() */
  LA_ERR_HIP = 4           /* a HIP runtime call or launch failed */
} la_status;

typedef enum {
  LA_BF16 = 0,             /* bfloat16 tokens; fp32 accumulation and states */
  LA_FP32 = 1              /* float32 everywhere */
} la_dtype;

/*
 * Problem shape.
 *   B, H, L   batch, heads, tokens per (b, h) sequence; B, H, L >= 0.
 *   dk, dv    head dimensions; this version needs dk == dv in {64, 128}.
 *   nseg      >= 1: each (b, h) sequence is cut into nseg consecutive
 *             segments of L / nseg tokens (L % nseg == 0) that are run
 *             independently, segment s starting from S0[b, h, s] and
 *             ending in S_end[b, h, s].  nseg = 1 is the plain call.
 *   dtype     la_dtype of the token tensors.
 *   split     internal sub-segments per segment used for parallelism
 *             (0 = the library's choice).  Any value gives the same result
 *             up to fp32 rounding; it exists for tuning and testing.
 *   reserved  must be 0.
 */
typedef struct {
  int64_t B, H, L;
  int32_t dk, dv;
  int32_t nseg;
  int32_t dtype;
  int32_t split;
  int32_t reserved;
} la_shape;

/* Library version (currently 1). */
int la_version(void);

/* Static string for a status code. */
const char* la_status_str(la_status status);

/* Message describing the last failed call on this thread ("" if none). */
const char* la_last_error(void);

/*
 * Workspace (device memory, 256-byte aligned) that la_chunk_fwd needs for
 * `shape`, in bytes; 0 means none.  Returns 0 for an invalid shape too (the
 * call itself then reports the error).
 */
size_t la_fwd_workspace_bytes(const la_shape* shape);

/*
 * Forward pass.
 *   Q, K [B,H,L,dk], V [B,H,L,dv]     inputs, required (unless B*H*L == 0).
 *   lambda [H]                         decay per head, required.
 *   S0 [B,H,nseg,dk,dv] fp32           initial state per segment; NULL = zero.
 *   O [B,H,L,dv]                       output; NULL = state only (no O).
 *   S_end [B,H,nseg,dk,dv] fp32        final state per segment; NULL = skip.
 *   ws, ws_bytes                       workspace of la_fwd_workspace_bytes().
 * O and S_end must not both be NULL.
 * Row (b, h, t) of O is o_t of segment s = t / (L/nseg) of sequence (b, h),
 * computed from S0[b, h, s].
 */
la_status la_chunk_fwd(const la_shape* shape, const void* Q, const void* K,
                       const void* V, const float* lambda, const float* S0,
                       void* O, float* S_end, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * Segment state-combine scan (fp32).  For every (b, h), with
 * a = lambda[h]^seg_len, X = S0[b, h] (or zero if S0 is NULL):
 *     for s = 0, 1, ..., P-1   (reverse != 0: s = P-1, ..., 0)
 *         S_start[b, h, s] = X;   X = a * X + dS[b, h, s]
 *     S_end[b, h] = X           (if S_end is not NULL)
 * dS are the per-segment local states (accumulated from zero over seg_len
 * tokens, e.g. by la_chunk_fwd with nseg = P, S0 = NULL, O = NULL); S_start
 * are then the initial states that make segmented runs equal one run: the
 * combine S_end = lambda^seg_len * S_start + dS of the All-Scan of ZeCO and of
 * the memory-state gather of LASP-2.  The reverse scan is the same combine
 * for gradient states flowing from the last segment to the first.
 *   dS [B,H,P,dk,dv]   S_start [B,H,P,dk,dv] (may be the same buffer as dS)
 *   S0, S_end [B,H,dk,dv]   lambda [H]   seg_len >= 0   P >= 0
 * lambda^seg_len is evaluated in fp32 as exp2(seg_len * log2(lambda)).
 */
la_status la_state_scan(int64_t B, int64_t H, int32_t P, int32_t dk, int32_t dv,
                        const float* dS, const float* lambda, int64_t seg_len,
                        const float* S0, float* S_start, float* S_end,
                        int32_t reverse, void* stream);

/* Workspace bytes la_chunk_bwd needs for `shape` (see la_fwd_workspace_bytes). */
size_t la_bwd_workspace_bytes(const la_shape* shape);

/*
 * Backward pass of la_chunk_fwd for the loss
 *     l = sum_t <dO_t, o_t> + <dS_end, S_end>
 * (per segment).  Gradients are exact for the recurrence above:
 *     dq_t = S_t dO_t
 *     dk_t = G_t v_t,  dv_t = G_t^T k_t,  with G_t = q_t dO_t^T + lambda G_{t+1}
 *            and lambda G_{L+1} = dS_end
 *     dS0  = lambda G_1
 *   Q, K, V, lambda, S0   as for la_chunk_fwd (S0 NULL = zero).
 *   dO [B,H,L,dv]         upstream gradient of O, required.
 *   dS_end                upstream gradient of S_end; NULL = zero.
 *   dQ, dK [B,H,L,dk], dV [B,H,L,dv]   outputs, required, dtype of the inputs.
 *   dS0 [B,H,nseg,dk,dv] fp32          output; NULL = not returned.
 *   ws, ws_bytes          workspace of la_bwd_workspace_bytes().
 * lambda receives no gradient here; la_decay_grad computes it.
 */
la_status la_chunk_bwd(const la_shape* shape, const void* Q, const void* K,
                       const void* V, const float* lambda, const float* S0,
                       const void* dO, const float* dS_end, void* dQ, void* dK,
                       void* dV, float* dS0, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * la_chunk_bwd for a training step that has just run la_chunk_fwd on the same
 * inputs: the dQ sweep takes the sub-segment start states that forward call
 * left in its workspace instead of recomputing them (a state pre-pass over K
 * and V and a scan: about one eighth of la_chunk_bwd's time at 256K tokens x
 * 16 heads).  The intermediate memory states are what the LASP-2 page's
 * abstract exchanges between ranks; keeping them from the forward is the
 * single-GPU form of that reuse.
 *   fwd_ws   the workspace of a la_chunk_fwd call with the same shape (split
 *            included), Q, K, V, lambda and S0, not written since; read only.
 *            Required when la_fwd_workspace_bytes(shape) > 0, else ignored.
 *   other arguments and the workspace as for la_chunk_bwd.
 * Results agree with la_chunk_bwd up to fp32 rounding (the forward forms the
 * same states with K and V in the other operand roles).  Errors as
 * la_chunk_bwd; a stale or foreign fwd_ws gives wrong numbers, not an error.
 */
la_status la_chunk_bwd_from_fwd(const la_shape* shape, const void* Q, const void* K,
                                const void* V, const float* lambda, const float* S0,
                                const void* dO, const float* dS_end, const void* fwd_ws,
                                void* dQ, void* dK, void* dV, float* dS0, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * Gated recurrence: the fixed decay becomes a per-token, per-head gate,
 *     S_t = alpha_t * S_{t-1} + k_t v_t^T        o_t = q_t^T S_t
 * the data-dependent gates of the "Gated Linear Attention Transformers with
 * Hardware-Efficient Training" entry of the LASP-2 page's related-paper
 * list, taken as one scalar gate per token and head.  Same chunkwise
 * evaluation as la_chunk_fwd with every lambda power replaced by a product
 * of gates (exp of a difference of chunk-local cumulative log-gates, all
 * <= 1); segments combine with the product of their gates.
 */

/* Workspace bytes la_chunk_fwd_gated needs for `shape`; 0 = none (or an
 * invalid shape). */
size_t la_fwd_gated_workspace_bytes(const la_shape* shape);

/*
 * Gated forward pass.  As la_chunk_fwd, with
 *   log_alpha [B,H,L] fp32   log of the gates, log(alpha_t) <= 0 (alpha_t in
 *                            (0, 1]); required (no lambda argument).
 * Segment s of (b, h) (nseg > 1) starts from S0[b, h, s] and uses the gates
 * of its own tokens only.  ws: workspace of la_fwd_gated_workspace_bytes().
 * Errors as la_chunk_fwd; nothing is written when validation fails.
 */
la_status la_chunk_fwd_gated(const la_shape* shape, const void* Q, const void* K,
                             const void* V, const float* log_alpha, const float* S0,
                             void* O, float* S_end, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * Gated segment combine: la_state_scan with the decay of segment s of (b, h)
 * given as its log, log_decay[b, h, s] (the sum of the segment's log-gates):
 *     S_start[b, h, s] = X;   X = exp(log_decay[b, h, s]) * X + dS[b, h, s]
 *   dS, S_start [B,H,P,dk,dv] (may be the same buffer)   log_decay [B,H,P] fp32
 *   S0, S_end [B,H,dk,dv] (S0 NULL = zero, S_end NULL = not written)
 * Errors as la_state_scan.
 */
la_status la_state_scan_gated(int64_t B, int64_t H, int32_t P, int32_t dk, int32_t dv,
                              const float* dS, const float* log_decay, const float* S0,
                              float* S_start, float* S_end, int32_t reverse, void* stream);

/* Workspace bytes la_chunk_bwd_gated needs for `shape`: about 3.4 (segments
 * of whole 64-token chunks) to 4.5 (ragged ones) times ceil(L/nseg / 1024)
 * fp32 d x d states per sequence (the sweeps' start states and the states at
 * every 1024th row, about 220 B per token-head at d = 128) plus the shifted
 * gates and per-token sums. */
size_t la_bwd_gated_workspace_bytes(const la_shape* shape);

/*
 * Backward pass of la_chunk_fwd_gated for the loss
 *     l = sum_t <dO_t, o_t> + <dS_end, S_end>   (per segment):
 *     dq_t = S_t dO_t
 *     dk_t = G_t v_t,  dv_t = G_t^T k_t,  G_t = q_t dO_t^T + alpha_{t+1} G_{t+1},
 *            alpha_{L+1} G_{L+1} = dS_end
 *     dS0  = alpha_1 G_1
 *     d l / d log(alpha_t) = alpha_t <G_t, S_{t-1}>
 *                          = sum_{u >= t} (q_u . dq_u - k_u . dk_u) + <dS_end, S_end>
 * (the second form, used here, holds because log(alpha_t) enters only through
 * the cumulative log-gates).
 *   Q, K, V, log_alpha, S0   as for la_chunk_fwd_gated (S0 NULL = zero).
 *   dO [B,H,L,dv] required; dS_end NULL = zero.
 *   dQ, dK, dV                outputs, required, dtype of the inputs.
 *   dS0 [B,H,nseg,dk,dv] fp32 output; NULL = not returned.
 *   dlog_alpha [B,H,L] fp32   output; NULL = not returned.
 *   ws, ws_bytes              workspace of la_bwd_gated_workspace_bytes().
 * The sweeps' start states are always formed at every 1024th row of each
 * segment (whatever shape->split asks for), the reverse ones counted from the
 * segment's end so that both fall on the same rows: at every such row y the
 * gate gradient alpha_y <G_y, S_{y-1}> is formed exactly from the two
 * sweeps' fp32 states, so the suffix sums of the second form never span more
 * than 1024 tokens.  The sweeps themselves walk whole multiples of 1024 tokens
 * (shape->split, rounded up; 0 = the library's choice).
 * Errors as la_chunk_bwd.
 */
la_status la_chunk_bwd_gated(const la_shape* shape, const void* Q, const void* K,
                             const void* V, const float* log_alpha, const float* S0,
                             const void* dO, const float* dS_end, void* dQ, void* dK,
                             void* dV, float* dS0, float* dlog_alpha, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * la_chunk_bwd_gated for a training step that has just run la_chunk_fwd_gated
 * on the same inputs, as la_chunk_bwd_from_fwd is for la_chunk_bwd: when the
 * backward's sweeps walk the forward's own sub-segments (the forward's plan
 * cuts each segment into whole 1024-token blocks, e.g. 8192-token
 * sub-segments, and the segments are whole 64-token chunks or dlog_alpha is
 * NULL), the dQ sweep takes the start states that forward call left in its
 * workspace instead of a gated state pre-pass over K and V and a scan (about
 * one ninth of the gated backward's time at 256K tokens x 16 heads).  Any
 * other shape forms them itself and does not read fwd_ws.
 *   fwd_ws   the workspace of a la_chunk_fwd_gated call with the same shape
 *            (split included), Q, K, V, log_alpha and S0, not written since;
 *            read only.  Required when la_fwd_gated_workspace_bytes(shape) > 0,
 *            else ignored.
 *   other arguments and the workspace as for la_chunk_bwd_gated.
 * Results agree with la_chunk_bwd_gated up to fp32 rounding (the forward
 * forms the same states with K and V in the other operand roles).  Errors as
 * la_chunk_bwd_gated; a stale or foreign fwd_ws gives wrong numbers, not an
 * error.
 */
la_status la_chunk_bwd_gated_from_fwd(const la_shape* shape, const void* Q, const void* K,
                                      const void* V, const float* log_alpha, const float* S0,
                                      const void* dO, const float* dS_end, const void* fwd_ws,
                                      void* dQ, void* dK, void* dV, float* dS0,
                                      float* dlog_alpha, void* ws, size_t ws_bytes,
                                      void* stream);

/* Workspace bytes la_decay_grad needs for `shape`; 0 for an invalid shape. */
size_t la_decay_grad_workspace_bytes(const la_shape* shape);

/*
 * Gradient of the loss of la_chunk_bwd with respect to the decays, for a
 * trainable lambda (the per-head decay rate of the Lightning Attention-2
 * entry of the LASP-2 page's related-paper list, there a fixed constant):
 *     d l / d lambda_h,   l = sum_t <dO_t, o_t> + <dS_end, S_end>
 * summed over every sequence (batch entry and segment) of head h.  Computed
 * by forward-mode differentiation: the tangent state T_t = d S_t / d lambda
 * obeys T_t = lambda T_{t-1} + S_{t-1}, T_0 = 0, and
 *     d l / d lambda = sum_t dO_t . (q_t^T T_t) + <dS_end, T_end>
 *                    = sum_t <G_t, S_{t-1}>     (G_t as in la_chunk_bwd).
 * The tangent walk is chunked like la_chunk_fwd (state and tangent fp32,
 * per-workgroup shares summed in fp64 in a fixed order).  It carries
 * lambda T and divides the final sum by lambda_h, so it needs lambda_h > 0
 * (and loses precision for lambda_h far below 1e-38, where lambda T falls
 * into the fp32 denormals).
 *   Q, K, V, lambda, S0, shape   as for la_chunk_fwd (S0 NULL = zero).
 *   dO [B,H,L,dv]                upstream gradient of O, required.
 *   dS_end [B,H,nseg,dk,dv] fp32 upstream gradient of S_end; NULL = zero.
 *   dlambda [H] fp32             output.
 *   ws, ws_bytes                 workspace of la_decay_grad_workspace_bytes().
 * Errors as la_chunk_bwd.
 */
la_status la_decay_grad(const la_shape* shape, const void* Q, const void* K,
                        const void* V, const float* lambda, const float* S0,
                        const void* dO, const float* dS_end, float* dlambda,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * One recurrent decode step for a batch of B * H sequences: the token
 * recurrence above applied to one new token per sequence (the
 * "constant-memory inference" of the LASP-2 page's abstract):
 *     S_out = lambda_h S + k v^T          o = q^T S_out
 *   q, k [B,H,dk], v [B,H,dv], o [B,H,dv]   element type `dtype`
 *                                           (LA_BF16 or LA_FP32).
 *   lambda [H] fp32.
 *   S, S_out [B,H,dk,dv] fp32   state before / after the token.  S NULL =
 *                               zero (a sequence's first token).  S_out may
 *                               be S itself (in place) but may not overlap
 *                               it otherwise.
 *   o                           output; NULL = state update only.
 * dk == dv in {64, 128}.  The state is read and written once (fp32
 * arithmetic throughout); o is rounded to `dtype`.  B * H == 0 is a no-op.
 * Errors as la_chunk_fwd.
 */
la_status la_step(int64_t B, int64_t H, int32_t dk, int32_t dv, int32_t dtype,
                  const void* q, const void* k, const void* v, const float* lambda,
                  const float* S, float* S_out, void* o, void* stream);

/*
 * One decode step of the gated recurrence (la_chunk_fwd_gated) for a batch
 * of B * H sequences, the token's own gate in place of lambda_h:
 *     S_out = alpha S + k v^T          o = q^T S_out
 *   log_alpha [B,H] fp32   log of the token's gate per sequence and head,
 *                          log(alpha) <= 0; required.  alpha is formed in
 *                          fp32 as 2^(log_alpha * log2 e).
 *   other arguments, checks and errors as la_step.
 * Stepping a sequence token by token from S0 gives la_chunk_fwd_gated's
 * outputs and final state over those tokens, up to rounding.
 */
la_status la_step_gated(int64_t B, int64_t H, int32_t dk, int32_t dv, int32_t dtype,
                        const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* S, float* S_out, void* o, void* stream);

/*
 * la_chunk_fwd without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and checks as la_chunk_fwd (the
 * same kernels, bit for bit), minus ws and ws_bytes: the start states of the
 * split plan live in a fixed device array of the library,
 * LA_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load on that GPU
 * until the process ends.  The call allocates and frees nothing.
 *  - A shape whose plan needs more than LA_NOALLOC_SCRATCH_BYTES
 *    (la_fwd_workspace_bytes) is rejected with LA_ERR_WORKSPACE before any
 *    HIP call, and nothing is written.  32 MiB covers, e.g., 32 heads of 64K
 *    tokens (14 MiB) and 16 heads of 256K tokens (31 MiB) at d = 128.
 *  - `stream` must belong to the current device (the array is per device).
 *  - Every call on one GPU shares that GPU's array: two calls that overlap in
 *    time on one GPU (on different streams or host threads) race and give
 *    wrong numbers.  Calls in one stream's order are safe.
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
la_status la_chunk_fwd_noalloc(const la_shape* shape, const void* Q, const void* K,
                               const void* V, const float* lambda, const float* S0,
                               void* O, float* S_end, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
