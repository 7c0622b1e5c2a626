/*
 * e2ttt.h -- C ABI of the E2-TTT chunk-parallel fast-weight update (gfx950).
 *
 * The operation is the chunk forward of "Rethinking Expressivity and
 * Efficiency in Test-Time Training" (E2-TTT):
 *   - per chunk of C tokens, every token's descent direction
 *     G_t = -grad_W 0.5*||f_W(k_t) - v_t||^2 is evaluated at the chunk-start
 *     fast weights W_0 (§1, §3; App. A.5);
 *   - the chunk-end pair (W_C, M_C) equals that of the token-wise recurrence
 *     M_t = beta_t M_{t-1} + eta_t G_t,  W_t = gamma_t W_{t-1} + M_t
 *     (Eq. 7 as read from §3.2 and App. A.5), reached through the two scalar
 *     kernels K^M_t = eta_t*beta~_t and K^W_t = eta_t*beta~_t*R_t of §3.2:
 *         M_C = cM*M_0 + sum_t K^M_t G_t
 *         W_C = cW*W_0 + cWM*M_0 + sum_t K^W_t G_t
 *     with beta~_t, gamma~_t the suffix products of beta and gamma over the
 *     chunk's later tokens (App. A.2 forms them in log space; here they are
 *     fp64 products of linear maps in a suffix scan, see
 *     e2ttt_scalar_kernels);
 *   - gamma_t = 1 - eta_t*alpha_t (Eq. 14, App. A.3), or gamma_t = alpha_t
 *     with E2TTT_ALPHA_IS_GAMMA;
 *   - the readout is o_t = f_{W_0}(q_t) with the chunk-start weights (Eq. 6);
 *   - (W_C, M_C) of one chunk is (W_0, M_0) of the next (§3.2, induction).
 *
 * Fast-weight learners (§2, §5.2, App. B.5):
 *   E2TTT_LINEAR : f_W(x) = W x, W is d x d row-major.
 *   E2TTT_SWIGLU : f(x) = W2 (silu(W1 x) * (W3 x)); the state of one
 *                  (batch, head) is packed [W1 (h x d) | W3 (h x d) | W2 (d x h)],
 *                  each row-major, P = 3*d*h floats.
 *   E2TTT_MLP    : f(x) = W2 silu(W1 x), the smaller fast-weight network of
 *                  E2-TTT_MLP (§5, App. B.3 Table 11, App. B.5; the page
 *                  names no activation: SiLU, the SwiGLU's, is taken);
 *                  packed [W1 (h x d) | W2 (d x h)], P = 2*d*h floats.  It
 *                  runs on the SwiGLU kernels with the gate branch held at
 *                  one (an internal copy of the state carries W3 = 0 and the
 *                  gate's pre-activation is replaced by 1, its gradient by
 *                  0).  Supported by every entry point; the states and
 *                  their adjoints at the boundary are always [W1 | W2].
 *
 * Layouts (all contiguous, row-major):
 *   q, k, v, out          [B, H, L, d]   io_dtype (fp32 or bf16)
 *   eta, alpha, beta      [B, H, L]      fp32
 *   W0, M0, W_end, M_end  [B, H, P]      fp32   (P = d*d, 3*d*h or 2*d*h)
 * Chunks are consecutive runs of C tokens from the start of the sequence; if
 * C does not divide L the last chunk is shorter (same recurrence, fewer
 * tokens).  L == 0 copies (W0, M0) to (W_end, M_end).
 *
 * Ownership and concurrency: every tensor pointer is a DEVICE pointer owned
 * by the caller; the library allocates nothing and keeps no state between
 * calls.  Work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns without synchronising.  Inputs are read only.
 * W_end may be exactly W0 and M_end exactly M0 (in-place state advance);
 * any other overlap between outputs, inputs or the workspace is EINVAL.
 *
 * Errors: every check runs on the host before anything is enqueued; on error
 * nothing is launched and nothing is written.  NaN/Inf in the inputs are
 * propagated, not detected.  No C++ exception crosses this interface.
 */
#ifndef E2TTT_H_
#define E2TTT_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define E2TTT_API __attribute__((visibility("default")))
#else
#define E2TTT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  E2TTT_OK = 0,
  E2TTT_EINVAL = 1,       /* bad pointer, size, alignment, overlap or flags */
  E2TTT_EWORKSPACE = 2,   /* workspace smaller than e2ttt_workspace_bytes() */
  E2TTT_EUNSUPPORTED = 3, /* shape/dtype outside the compiled kernels */
  E2TTT_EHIP = 4          /* a HIP runtime call or kernel launch failed */
} e2ttt_status;

typedef enum { E2TTT_LINEAR = 0, E2TTT_SWIGLU = 1, E2TTT_MLP = 2 } e2ttt_fast_weight;
typedef enum { E2TTT_F32 = 0, E2TTT_BF16 = 1 } e2ttt_dtype;
typedef enum {
  E2TTT_GAMMA_1_MINUS_ETA_ALPHA = 0, /* gamma = 1 - eta*alpha (Eq. 14) */
  E2TTT_ALPHA_IS_GAMMA = 1           /* gamma = alpha                  */
} e2ttt_decay_mode;

/* Bits of e2ttt_problem.flags.
 *
 * Precision of the fast-weight operands (SwiGLU, bf16 io).  The matrix cores
 * take bf16 operands; the fast weights are fp32.  A weight rounded to bf16
 * carries 8 mantissa bits; a hi/lo pair (W = hi + lo, both multiplied against
 * the same activations) carries ~16.  By default, with d = 128, the products
 * that feed the chunk-end state (the recomputed W1 x, W3 x and the W2^T g of
 * the backward at W_0) use the hi/lo pair and the readout's forward uses hi
 * only: the state's error per chunk is then ~1.6e-3 instead of ~2.4e-3,
 * which matters when every chunk rebuilds the state from gradients that are
 * polynomial in W_0, so that relative errors roughly double from chunk to
 * chunk.  The other shapes use plain bf16 weights unless the
 * compensated flag is set. */
enum {
  /* SwiGLU with bf16 io: the hi/lo pair in every forward and backward
   * product (the readout's too), at about 1.7x the matrix-core work of
   * plain bf16 weights.  Ignored for fp32 io and LINEAR. */
  E2TTT_FLAG_COMPENSATED_WEIGHTS = 1u,
  /* The chunk-averaged variant ("Rethinking Expressivity and Efficiency in
   * Test-Time Training", §5.4 Table 5 and App. B.3 Table 8): within each
   * chunk the per-token momentum factors beta_t and decay factors gamma_t
   * (after decay_mode) are replaced by their arithmetic means over the
   * chunk's tokens before the scalar kernels are formed; eta_t stays per
   * token.  Applies to e2ttt_chunk_forward, its timed twin,
   * e2ttt_scalar_kernels, e2ttt_decode_step (the means over the buffered
   * tokens at each chunk end) and the backward, for every kind and dtype. */
  E2TTT_FLAG_CHUNK_AVERAGED_DECAY = 2u,
  /* The TTT branch's input prologue ("Rethinking Expressivity and
   * Efficiency in Test-Time Training", §4 Overall Architecture): q and k are
   * passed as raw projections, and the library applies SiLU and then L2
   * normalisation to every token's vector (x / max(||x||, 1e-12), in fp32,
   * rounded to io_dtype) before using them.  Applies to e2ttt_chunk_forward,
   * its timed twin, e2ttt_decode_step and the backward (which takes dq, dk
   * back through it); the workspace grows by the two normalised copies. */
  E2TTT_FLAG_QK_SILU_L2 = 4u,
  /* Chunk-boundary normalisation of the fast weights ("Rethinking
   * Expressivity and Efficiency in Test-Time Training", App. B.1 Training
   * Details, a stabiliser taken over from LaCT): after every chunk's update,
   * the last one included, each row of each fast-weight matrix (linear W;
   * SwiGLU W1, W3, W2, rows as stored) is divided by max(||row||_2, 1e-12),
   * in fp32 with a fixed summation order.  M is not changed.  The next
   * chunk's readout and descent directions use the normalised W.  Applies to
   * e2ttt_chunk_forward, its timed twin and e2ttt_decode_step (at a call with
   * chunk_end set), and the backward (through every normalisation). */
  E2TTT_FLAG_POST_CHUNK_ROW_L2 = 8u,
  /* SwiGLU with bf16 io and d = 128: plain bf16 fast-weight operands in every
   * product (the fastest setting; ~2.4e-3 relative error on the chunk-end
   * state per chunk).  Exclusive with E2TTT_FLAG_COMPENSATED_WEIGHTS
   * (EINVAL when both are set); no effect on other shapes, fp32 io, LINEAR,
   * the decode step and the backward, which use their weights in fp32. */
  E2TTT_FLAG_PLAIN_BF16_WEIGHTS = 16u,
  /* The LaCT rule ("Rethinking Expressivity and Efficiency in Test-Time
   * Training", §3.2 "Two scalar kernels with distinct temporal weighting",
   * Eq. 5, and §1): one update per chunk from the eta-weighted sum of the
   * chunk's descent directions, with the momentum and decay factors
   * collapsed to their chunk means:
   *     M_C = mean(beta) M_0 + sum_t eta_t G_t,  W_C = mean(gamma) W_0 + M_C
   * (gamma after decay_mode; G_t at W_0; readout as the default).  The
   * display of Eq. 5 is missing from the page; this is the reading of its
   * description there (no momentum suffix product, no decay ratio sum).
   * Same kernels as the default rule, only the scalar kernels differ:
   * K^W = K^M = eta, (cW, cM, cWM) = (mean gamma, mean beta, mean beta).
   * Applies to e2ttt_chunk_forward (and its twins), e2ttt_scalar_kernels,
   * e2ttt_decode_step (the update at each chunk end) and the backward (deta
   * takes the adjoints of both kernels; each token's beta and gamma get 1/n
   * of the adjoints of the means); EINVAL together with
   * E2TTT_FLAG_CHUNK_AVERAGED_DECAY. */
  E2TTT_FLAG_LACT_RULE = 32u
};

/* Problem description.  struct_size must equal sizeof(e2ttt_problem). */
typedef struct {
  uint32_t struct_size;
  int32_t kind;       /* e2ttt_fast_weight */
  int64_t batch;      /* B >= 1 */
  int64_t heads;      /* H >= 1 */
  int64_t seq_len;    /* L >= 0 */
  int64_t dim;        /* d >= 1 */
  int64_t hidden;     /* h (SwiGLU); must be 0 for LINEAR */
  int64_t chunk;      /* C >= 1 */
  int32_t io_dtype;   /* e2ttt_dtype of q, k, v, out; states are fp32 */
  int32_t decay_mode; /* e2ttt_decay_mode */
  uint32_t flags;     /* E2TTT_FLAG_* bits; others must be 0 */
  uint32_t reserved;  /* must be 0 */
} e2ttt_problem;

/* Host-only argument check (no HIP call).  Returns E2TTT_OK if the problem is
 * well formed and supported:
 *   LINEAR : 16 <= d <= 128, d % 16 == 0, io fp32 or bf16.
 *   SWIGLU, MLP : d % 128 == 0, h % 128 == 0, d <= 1024, h <= 4096, io fp32 or bf16.
 *   Both   : 1 <= C <= 12288.
 * EINVAL for malformed values, EUNSUPPORTED for well-formed but uncompiled. */
E2TTT_API e2ttt_status e2ttt_validate(const e2ttt_problem* prob);

/* Host-only: bytes of device workspace e2ttt_chunk_forward needs for `prob`
 * (written to *bytes).  The workspace must be 256-byte aligned. */
E2TTT_API e2ttt_status e2ttt_workspace_bytes(const e2ttt_problem* prob, size_t* bytes);

/* The chunk forward over the whole sequence (all B*H units, all chunks).
 * Inputs: q, k, v [B,H,L,d] io_dtype; eta, alpha, beta [B,H,L] fp32;
 * W0, M0 [B,H,P] fp32.  Outputs: out [B,H,L,d] io_dtype, W_end, M_end
 * [B,H,P] fp32 (the state after the last chunk).  workspace: device memory
 * of at least e2ttt_workspace_bytes() bytes, 256-byte aligned, not
 * overlapping anything else; its contents are scratch.  All tensor pointers
 * must be 16-byte aligned.  Enqueued on `stream`; returns E2TTT_EHIP if a
 * launch fails (asynchronous faults surface at the caller's next sync). */
E2TTT_API e2ttt_status e2ttt_chunk_forward(const e2ttt_problem* prob, const void* q,
                                 const void* k, const void* v,
                                 const float* eta, const float* alpha,
                                 const float* beta, const float* W0,
                                 const float* M0, void* out, float* W_end,
                                 float* M_end, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* e2ttt_chunk_forward that also keeps, for training, the state each chunk
 * starts from (the chunk-to-chunk carry of §3.2: (W_C, M_C) of chunk r is the
 * start of chunk r+1), so that e2ttt_chunk_backward_states need not recompute
 * them.  W_starts, M_starts: [nC-1][B,H,P] fp32 (nC = ceil(L / chunk)); slot
 * r - 1 holds the state at the start of chunk r, after the chunk-boundary
 * normalisation when that flag is set.  Both must be non-null, 16-byte aligned
 * and overlap nothing else when nC > 1 (EINVAL); with nC <= 1 they are not
 * touched.  Everything else as e2ttt_chunk_forward, same workspace. */
E2TTT_API e2ttt_status e2ttt_chunk_forward_states(const e2ttt_problem* prob, const void* q,
                                                  const void* k, const void* v,
                                                  const float* eta, const float* alpha,
                                                  const float* beta, const float* W0,
                                                  const float* M0, void* out, float* W_end,
                                                  float* M_end, float* W_starts,
                                                  float* M_starts, void* workspace,
                                                  size_t workspace_bytes, void* stream);

/* e2ttt_chunk_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, results and checks as e2ttt_chunk_forward,
 * minus the workspace: the call uses a scratch array of
 * E2TTT_NOALLOC_SCRATCH_BYTES built into the library, one per GPU (each GPU
 * holds it from the library's load until the process ends), and calls no
 * allocating routine.  Problems whose e2ttt_workspace_bytes() exceeds that
 * size return E2TTT_EWORKSPACE (nothing launched).  The array is shared by
 * every call on one GPU and keeps the last call's contents (the forward
 * treats it as uninitialised scratch): calls that may overlap in time on one
 * GPU, on different streams or from different threads, race and must be
 * serialised by the caller.  The device address of a GPU's array is looked
 * up at the first call on that GPU (E2TTT_EHIP if that fails). */
#define E2TTT_NOALLOC_SCRATCH_BYTES (64u << 20)
E2TTT_API e2ttt_status e2ttt_chunk_forward_noalloc(const e2ttt_problem* prob, const void* q,
                                                   const void* k, const void* v,
                                                   const float* eta, const float* alpha,
                                                   const float* beta, const float* W0,
                                                   const float* M0, void* out, float* W_end,
                                                   float* M_end, void* stream);

/* The per-token scalar kernels alone (§3.2, App. A.2-A.3), for every chunk:
 *   k_w[b,h,t] = K^W_t = eta_t * beta~_t * R_t  (weight kernel)
 *   k_m[b,h,t] = K^M_t = eta_t * beta~_t        (momentum kernel)
 *   chunk_coef[b,h,r,0..2] = (cW, cM, cWM): the factors of W_0 in W_C, of
 *   M_0 in M_C and of M_0 in W_C for chunk r.
 * beta~_t is the product of beta_s over the later tokens s > t of the chunk;
 * R_t sums the ratios gamma~_i / beta~_i over i >= t.  The ratio sum is never
 * formed: beta~_t R_t is evaluated as the bounded recursion
 * P_t = gamma~_t + beta_{t+1} P_{t+1}, P_last = 1, in fp64.
 * Shapes: eta, alpha, beta, k_w, k_m [B,H,L] fp32; chunk_coef [B,H,nC,3]
 * fp32 with nC = ceil(L/C).  Only batch, heads, seq_len, chunk and
 * decay_mode of `prob` are used (kind/dim/hidden/io_dtype are still
 * validated).  Pointers 16-byte aligned except chunk_coef (4-byte). */
E2TTT_API e2ttt_status e2ttt_scalar_kernels(const e2ttt_problem* prob, const float* eta,
                                  const float* alpha, const float* beta,
                                  float* k_w, float* k_m, float* chunk_coef,
                                  void* stream);

/* The per-token scalar heads of the TTT branch ("Rethinking Expressivity
 * and Efficiency in Test-Time Training", §4 Overall Architecture and
 * Input-Dependent Dynamics; App. B.3, B.4): linear heads on the layer input
 * give the inputs eta, alpha, beta of e2ttt_chunk_forward.  For token t of
 * batch b and TTT head h (H = prob->heads):
 *   eta[b,h,t]   = eta_base   * sigmoid(<w_heads[h],      x[b,t]> + b_heads[h])
 *   alpha[b,h,t] = alpha_base * sigmoid(<w_heads[H + h],  x[b,t]> + b_heads[H + h])
 *   beta[b,h,t]  =              sigmoid(<w_heads[2H + h], x[b,t]> + b_heads[2H + h])
 * (App. B.3: the base scalars scale the sigmoid gates; Eq. 13, beta's
 * timescale form, is missing from the page and taken as a plain sigmoid
 * gate; gamma follows from eta and alpha downstream by Eq. 14.)
 * x [B, L, model_dim] and w_heads [3H, model_dim] are of io_dtype, b_heads
 * [3H] fp32; eta, alpha, beta [B, H, L] fp32 (the layout the forward takes).
 * The products accumulate in fp32 on the matrix cores; x is read once for
 * all heads.  Only batch, heads, seq_len and io_dtype of `prob` are used
 * (the rest must validate).  Supported: model_dim a multiple of 64 in
 * [64, 65536], H <= 64 (else EUNSUPPORTED).  x and w_heads 16-byte aligned,
 * the rest 4-byte aligned; outputs must not overlap each other or the inputs
 * (EINVAL).  L = 0 does nothing.  Asynchronous on `stream`. */
E2TTT_API e2ttt_status e2ttt_scalar_heads(const e2ttt_problem* prob, const void* x,
                                          int64_t model_dim, const void* w_heads,
                                          const float* b_heads, float eta_base,
                                          float alpha_base, float* eta, float* alpha,
                                          float* beta, void* stream);

/* Kernel classes of the chunk forward, for e2ttt_chunk_forward_timed. */
typedef enum {
  E2TTT_KERNEL_SCAN = 0,       /* scalar kernels, all chunks (one launch)    */
  E2TTT_KERNEL_PREP = 1,       /* K^T staging (on the 256-tile path: the keys
                                  scaled by K^W and K^M) and W0 operand
                                  shadow                                    */
  E2TTT_KERNEL_FWD13 = 2,      /* [K;Q] x [W1;W3]^T -> Z (per chunk)          */
  E2TTT_KERNEL_FWD2 = 3,       /* Z x W2^T -> readout, g (per chunk)         */
  E2TTT_KERNEL_BWD = 4,        /* g x W2 -> dA1, dA3 (per chunk)             */
  E2TTT_KERNEL_AGG = 5,        /* scaled aggregations (+ state, unless split)
                                  (per chunk)                               */
  E2TTT_KERNEL_LINEAR_FWD = 6, /* linear learner: readout and residuals      */
  E2TTT_KERNEL_LINEAR_AGG = 7, /* linear learner: aggregations + state       */
  E2TTT_KERNEL_PHASE_A = 8,    /* d = 128 bf16: fused forward, readout, g     */
  E2TTT_KERNEL_PHASE_B = 9,    /* d = 128 bf16: fused backward, aggregations,
                                  chunk-end state (unless token-split)      */
  E2TTT_KERNEL_STATE = 10,     /* sum of the token splits (d = 128 bf16
                                  token-split phase B, or the split 256x256
                                  aggregation), chunk-end state, shadows    */
  E2TTT_KERNEL_PROLOGUE = 11,  /* d = 128 bf16: scalar kernels, K^T staging
                                  and W0 shadow in one launch               */
  E2TTT_KERNEL_NUM_CLASSES = 12
} e2ttt_kernel_class;

/* Benchmark instrumentation: enqueue exactly the work of e2ttt_chunk_forward
 * (same arguments, same results) and additionally record caller-created HIP
 * events (hipEvent_t, passed as void*) on every launch of one kernel class:
 * events[2j] at the start and events[2j+1] at the end of the j-th launch of
 * that class, for j < n_events/2 (recorded with the kernel dispatch itself,
 * so the elapsed time is the kernel's execution without the dispatch
 * latency).  *n_recorded (may be NULL) receives the number of launches
 * timed.  The caller reads the elapsed times after synchronising.  Same
 * error behaviour as e2ttt_chunk_forward; EINVAL for a bad kernel_class or
 * n_events < 0. */
E2TTT_API e2ttt_status e2ttt_chunk_forward_timed(const e2ttt_problem* prob, const void* q,
                                       const void* k, const void* v,
                                       const float* eta, const float* alpha,
                                       const float* beta, const float* W0,
                                       const float* M0, void* out, float* W_end,
                                       float* M_end, void* workspace,
                                       size_t workspace_bytes, void* stream,
                                       int kernel_class, void* const* events,
                                       int n_events, int* n_recorded);

/* Static, human-readable name of a status code. */
E2TTT_API const char* e2ttt_status_string(e2ttt_status status);

/* Streaming / decode use ("Rethinking Expressivity and Efficiency in
 * Test-Time Training": readout at the chunk-start weights, Eq. 6 and §3.2;
 * gradients at the chunk-start weights, §1 and §3; the chunk-end pair of the
 * token recurrence by the closed form, §3.2 and App. A; App. B.5: the
 * per-chunk bookkeeping is amortised over the chunk's tokens).  One call
 * processes ONE token of every (b, h) unit, the token at position `pos` of
 * the current chunk (0 <= pos < prob->chunk):
 *   out = f_W(q) with W the chunk-start weights;
 *   the token's descent factors at W, its key and its scalars are buffered
 *   in the workspace, slot pos;
 *   at a call with chunk_end != 0 the buffered tokens 0 .. pos are applied
 *   at once: (W, M) <- (W_C, M_C) of the chunk recurrence
 *     M <- beta M + eta G,  W <- gamma W + M  (gamma by decay_mode)
 *   exactly as e2ttt_chunk_forward forms them (scalar kernels, then the two
 *   weighted aggregations, fp32), then the chunk-boundary row normalisation
 *   when that flag is set.
 * So between chunk ends W and M hold the state at the chunk's start.  Calling
 * it for the tokens of a sequence in order, pos = t mod C, with chunk_end on
 * every C-th token and on the last, gives the outputs and end states of
 * e2ttt_chunk_forward on that sequence (up to rounding).  chunk_end must be
 * set at pos = C - 1 (EINVAL otherwise).  The workspace carries the chunk's
 * buffered tokens from call to call: every call of a chunk must get the same
 * workspace, unmodified; its size (e2ttt_decode_workspace_bytes) grows with
 * the chunk length: (7h + 4d + 5) floats per slot and unit for SwiGLU,
 * (4d + 5) for the linear learner.
 * Per token the call reads W (about 4P bytes) and writes a few vectors; the
 * full state is read and written once per chunk.
 * Shapes: q, k, v, out [B,H,d] io_dtype (this token); eta, alpha, beta [B,H]
 * fp32; W, M [B,H,P] fp32, updated in place at a chunk end.  Used from `prob`:
 * batch, heads, dim, hidden, chunk, kind, io_dtype, decay_mode and the flags
 * (seq_len must still validate).  With E2TTT_FLAG_CHUNK_AVERAGED_DECAY or
 * E2TTT_FLAG_LACT_RULE the chunk-end update takes the means over the
 * buffered tokens, as the chunk forward does over a chunk's tokens.  The
 * weight precision flags have no effect (fp32 throughout).  W, M, out and the
 * workspace must not overlap one another or the inputs (EINVAL).  All tensor
 * pointers 16-byte aligned, the workspace 256-byte aligned with at least
 * e2ttt_decode_workspace_bytes() bytes (EWORKSPACE).  Asynchronous on
 * `stream`; nothing is launched when an argument check fails. */
E2TTT_API e2ttt_status e2ttt_decode_workspace_bytes(const e2ttt_problem* prob, size_t* bytes);
E2TTT_API e2ttt_status e2ttt_decode_step(const e2ttt_problem* prob, const void* q,
                                         const void* k, const void* v, const float* eta,
                                         const float* alpha, const float* beta, float* W,
                                         float* M, void* out, int64_t pos, int chunk_end,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Outer-loop backward of e2ttt_chunk_forward (the gradients a model needs to
 * train through the chunk update; the throughput claims of B.5 "Throughput
 * and Inference Cost" of the E2-TTT paper are training throughput).  Given
 * the same inputs as the forward and the gradients dout = dl/dout, dW_end =
 * dl/dW_end, dM_end = dl/dM_end of a scalar loss l, it writes dl/dq, dl/dk,
 * dl/dv, dl/deta, dl/dalpha, dl/dbeta, dl/dW0, dl/dM0 through the whole chunk
 * recurrence: the readout at the chunk-start weights (Eq. 6), the per-token
 * descent directions at those weights (§3), the two weighted aggregations and
 * the chunk coefficients (§3.2, App. A), the scalar kernels' suffix products
 * and the affine reverse scan (App. A.2), and the decay coupling of Eq. 14
 * (or alpha taken as gamma).  Chunk-end states of every chunk are recomputed
 * by a forward pass inside the call.
 *
 * For the SwiGLU and MLP learners the descent direction depends on the
 * chunk-start weights through the learner (§5.2, App. B.5), so its reverse
 * mode carries the second-order terms of f = W2 (silu(W1 x) * (W3 x)) (or of
 * W2 silu(W1 x)) as well; the MLP learner's is the SwiGLU one with the gate
 * held at one, on an internal [W1 | 0 | W2] copy of the states and adjoints.
 *
 * Flags: E2TTT_FLAG_QK_SILU_L2 (the prologue is recomputed and dq, dk are
 * taken back through it to the raw q, k), E2TTT_FLAG_CHUNK_AVERAGED_DECAY
 * (each token's beta and gamma receive 1/n of the adjoints of its chunk's
 * means), E2TTT_FLAG_LACT_RULE (deta takes dK^W + dK^M, the means' adjoints
 * shared out as for the averaged variant), E2TTT_FLAG_POST_CHUNK_ROW_L2 (the adjoint goes back through every
 * chunk's normalisation; the states are then always recomputed, so
 * e2ttt_chunk_backward_states returns EUNSUPPORTED for it) and
 * E2TTT_FLAG_COMPENSATED_WEIGHTS (no effect: the arithmetic is fp32).
 * Supported: kind E2TTT_LINEAR
 * with dim a multiple of 16 up to 64, or E2TTT_SWIGLU / E2TTT_MLP with the
 * forward's (dim, hidden) set and at most 65535 batch*heads units (else
 * EUNSUPPORTED).  The arithmetic is fp32 (the forward
 * re-run too); with io_dtype E2TTT_BF16, q, k, v, dout are widened on entry
 * and dq, dk, dv rounded to nearest even on exit.  Layouts as the forward: q,
 * k, v, dout, dq, dk, dv [B,H,L,dim] of io_dtype; eta, alpha, beta,
 * deta, dalpha, dbeta [B,H,L]; W0, M0, dW_end, dM_end, dW0, dM0 [B,H,P] packed
 * as the forward's state (P = dim*dim, 3*dim*hidden or 2*dim*hidden).  dW_end and
 * dM_end may be NULL (zero gradients).  All pointers are device pointers owned
 * by the caller, 16-byte aligned (workspace 256); inputs are read-only; no
 * output may overlap another output, the workspace or any input (EINVAL).
 * L = 0 writes dW0 = dW_end, dM0 = dM_end only.  The workspace holds at least
 * e2ttt_backward_workspace_bytes() bytes (EWORKSPACE).  Asynchronous on
 * `stream`; nothing is launched when an argument check fails.  Sums over
 * tokens and state blocks run in a fixed order, so repeated calls give
 * identical bits. */
E2TTT_API e2ttt_status e2ttt_backward_workspace_bytes(const e2ttt_problem* prob,
                                                      size_t* bytes);
E2TTT_API e2ttt_status e2ttt_chunk_backward(const e2ttt_problem* prob, const void* q,
                                            const void* k, const void* v, const float* eta,
                                            const float* alpha, const float* beta,
                                            const float* W0, const float* M0, const void* dout,
                                            const float* dW_end, const float* dM_end, void* dq,
                                            void* dk, void* dv, float* deta, float* dalpha,
                                            float* dbeta, float* dW0, float* dM0,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/* e2ttt_chunk_backward given the chunk-start states kept by
 * e2ttt_chunk_forward_states for the same problem and inputs (read-only, must
 * not overlap an output; EINVAL when only one of the two is null).  The
 * forward re-run is skipped; the gradients are those of the forward whose
 * states were kept (for bf16 io that is the bf16 forward, rather than the fp32
 * re-run).  Both null: identical to e2ttt_chunk_backward.  Same workspace. */
E2TTT_API e2ttt_status e2ttt_chunk_backward_states(const e2ttt_problem* prob, const void* q,
                                                   const void* k, const void* v,
                                                   const float* eta, const float* alpha,
                                                   const float* beta, const float* W0,
                                                   const float* M0, const float* W_starts,
                                                   const float* M_starts, const void* dout,
                                                   const float* dW_end, const float* dM_end,
                                                   void* dq, void* dk, void* dv, float* deta,
                                                   float* dalpha, float* dbeta, float* dW0,
                                                   float* dM0, void* workspace,
                                                   size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* E2TTT_H_ */
