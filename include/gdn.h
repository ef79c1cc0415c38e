/*
 * libgdn -- the gated delta rule on AMD MI355X (gfx950), C ABI.
 *
 * Operation ("Gated Delta Networks: Improving Mamba2 with Delta Rule", paper
 * review, section "Method"): for every sequence and head, token by token,
 *
 *     S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 *
 * with S_t of shape dv x dk.  The library stores the state transposed,
 * M = S^T, as a row-major [dk, dv] fp32 matrix per (sequence, head).
 *   - alpha_t arrives as log alpha_t (finite, normally <= 0).  GDN_GATE_SCALAR
 *     takes one value per (token, head); GDN_GATE_CHANNEL one value per
 *     (token, head, key channel), which scales the dk rows of M (the
 *     Kimi-Delta-style diagonal gate that "Linear Attention Architectures:
 *     Mechanisms, Trade-offs, and Cross-Layer Routing" names); GDN_GATE_NONE
 *     is alpha = 1, the plain delta rule ("Key idea": alpha -> 1 recovers it).
 *   - beta_t is used as given (never clamped); q and k are used as given (the
 *     caller normalises them); there is no 1/sqrt(dk) scale.
 *   - The output reads the state after the token's own update.
 *
 * Three entry points:
 *   gdn_chunk_fwd   chunkwise-parallel forward over whole sequences (the WY /
 *                   UT-transform form named in "Method"), for prefill and
 *                   training;
 *   gdn_chunk_bwd   gradients of <dO, o> + <dS_final, S_final>;
 *   gdn_decode_step one token per sequence, updating the state in place
 *                   (the O(1)-memory recurrent inference of "Background").
 *
 * Conventions shared by all entry points
 *   Pointers: device pointers owned by the caller (e.g. torch tensors),
 *     contiguous, 16-byte aligned.  The library keeps no pointer after it
 *     returns and allocates no device memory: gdn_chunk_fwd / gdn_chunk_bwd
 *     take a caller-provided workspace of the size the *_workspace query
 *     returns.  Outputs must not alias inputs, except `state` of decode.
 *   Layouts (token-major, row-major):
 *     q, k       [B, T, H, dk]           (varlen: B = 1, T = total tokens)
 *     v, o, dO   [B, T, H, dv]
 *     beta       [B, T, H]
 *     log_alpha  [B, T, H] scalar gate, [B, T, H, dk] channel gate,
 *                ignored (may be NULL) for GDN_GATE_NONE
 *     s0, s_final, ds_final, ds0   [nseq, H, dk, dv] fp32
 *                (nseq = B for dense batches, the varlen sequence count else)
 *   Dtypes: q, k, v, o, dO, dq, dk, dv use io_dtype (fp32 or bf16); beta
 *     and log_alpha use gate_dtype; states, dbeta and dlog_alpha are fp32.
 *     bf16 operands are multiplied on the matrix cores with fp32
 *     accumulation; the state is always carried in fp32.
 *   Sizes: dk in {16, 32, 64, 128}; dv a multiple of 16 up to 256; chunk in
 *     {16, 32, 64}; H >= 1; T >= 0 (T = 0 is a no-op that copies s0 to
 *     s_final); B >= 1.
 *   Varlen: nseq > 0 with B == 1 packs nseq sequences; cu_seqlens is a
 *     DEVICE int32 array [nseq + 1] with cu_seqlens[0] = 0, non-decreasing,
 *     cu_seqlens[nseq] = T.  Its contents are a precondition (they are not
 *     read on the host); sequences of length 0 are allowed.  Chunks never
 *     cross a sequence boundary.
 *   Streams: all work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) with no implicit synchronisation.  The compute functions keep
 *     no state between calls: everything a call depends on is in its
 *     arguments, so they are re-entrant and may run concurrently on several
 *     streams (with separate workspaces).  The only process-wide settings
 *     are the two diagnostic hooks at the end of this header (stage timing
 *     and the launch-failure test hook), which change no result.
 *   Errors: every argument is validated on the host before anything is
 *     enqueued, so a non-OK status means nothing was launched.  A failed
 *     launch returns GDN_ERR_HIP.  Device faults surface at the caller's
 *     next synchronisation (asynchronous HIP semantics).  No function
 *     aborts or lets an exception escape.
 *   Diagnostics: the library writes nothing unless the environment variable
 *     GDN_LOG is set to a non-empty value other than "0" (read at every
 *     call).  Then each refused call writes one line to stderr with the
 *     entry point, the status and the source line of the failed check, and
 *     each launch writes the resolved problem and its dispatch choices
 *     (chunk count, segment length and count, steps per token, the
 *     normalising and write-strength variants) with the launch's HIP status.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 8

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL                     */
  GDN_ERR_SHAPE = 2,       /* a size is out of range or inconsistent         */
  GDN_ERR_DTYPE = 3,       /* unknown dtype code                              */
  GDN_ERR_UNSUPPORTED = 4, /* valid request outside the supported set        */
  GDN_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                */
  GDN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required      */
  GDN_ERR_HIP = 7,         /* the HIP runtime refused a launch                */
  GDN_ERR_SCRATCH = 8      /* gdn_chunk_fwd_noalloc: the problem needs more
                              workspace than the static scratch buffer holds */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum {
  GDN_GATE_NONE = 0,       /* alpha = 1: the delta rule without decay          */
  GDN_GATE_SCALAR = 1,     /* one log alpha per (token, head)                  */
  GDN_GATE_CHANNEL = 2     /* one log alpha per (token, head, key channel)     */
} gdn_gate;

/* Problem description.  For decode, T is ignored, B is the number of
 * sequences N and chunk / nseq / cu_seqlens / seg_chunks are ignored.
 *
 * seg_chunks: segment length of the state pass of the chunked forward (and
 * of the backward's state recompute).  The state is carried across the
 * chunks of each sequence; when there are few (sequence, head) pairs the
 * sequences are cut into segments of seg_chunks chunks, every segment's
 * affine state map is computed in parallel, the maps are chained in a short
 * sequential pass and the segments then run in parallel from their entering
 * states (the same recurrence, rounded differently).
 *   0  : automatic: segments long enough that the segment workgroups about
 *        fill the GPU's 256 compute units once and at least
 *        sqrt(chunks / 2.56) chunks; no split when the (sequence, head)
 *        pairs already fill the GPU or a sequence has fewer than 8 chunks;
 *   >0 : segments of seg_chunks chunks (values above 2^20 are clamped);
 *   <0 : never split.
 * It changes the workspace size: query the *_workspace function with the
 * same problem.  Draft trees ignore it (one chunk per tree). */
typedef struct {
  int32_t B, T, H, dk, dv, chunk;
  int32_t nseq;                 /* 0 = dense [B, T]; > 0 = varlen, B == 1     */
  const int32_t* cu_seqlens;    /* device [nseq + 1] when nseq > 0, else NULL */
  int32_t io_dtype;             /* gdn_dtype of q, k, v, o (and grads)        */
  int32_t gate_dtype;           /* gdn_dtype of beta and log_alpha            */
  int32_t gate;                 /* gdn_gate                                   */
  int32_t seg_chunks;           /* state-pass segment length, 0 = automatic   */
} gdn_problem;

/* ABI version of the loaded library (GDN_ABI_VERSION). */
int gdn_abi_version(void);

/* Static, never NULL, human-readable name of a status.  Takes the status as
 * an int so that any value is defined behaviour ("GDN_ERR_UNKNOWN" for values
 * outside gdn_status). */
const char* gdn_status_str(int status);

/* Workspace bytes gdn_chunk_fwd needs for problem *p (written to *bytes).
 * Returns the same validation status gdn_chunk_fwd would for the sizes. */
gdn_status gdn_chunk_fwd_workspace(const gdn_problem* p, size_t* bytes);

/* Chunkwise forward ("Method": the WY representation and UT transform keep
 * the recurrence in matrix-multiply form).  Per chunk of `chunk` tokens it
 * forms the chunk-local cumulative log-gate, the unit lower-triangular
 * system (I + tril(diag(beta) K K^T * decay, -1)) and its inverse T, the
 * WY factors W = T diag(beta * gamma) K and U = T diag(beta) V, then carries
 * the fp32 state across chunks.
 *   q, k, v, beta, log_alpha : inputs as in the header comment.
 *   s0      : initial state [nseq, H, dk, dv] fp32, or NULL for zeros.
 *   o       : output [B, T, H, dv] in io_dtype.
 *   s_final : final state [nseq, H, dk, dv] fp32, or NULL to skip it.
 *   ws      : device workspace of at least gdn_chunk_fwd_workspace bytes
 *             (256-byte aligned); contents on entry do not matter.
 */
gdn_status gdn_chunk_fwd(const gdn_problem* p, const void* q, const void* k,
                         const void* v, const void* beta,
                         const void* log_alpha, const float* s0, void* o,
                         float* s_final, void* ws, size_t ws_bytes,
                         void* stream);

/* The forward without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid allocation.  Computes exactly what
 * gdn_chunk_fwd computes (the same kernels, bit-identical results) but takes
 * its workspace from a static device array of GDN_NOALLOC_SCRATCH_BYTES
 * inside the library instead of from the caller.
 *   - Each GPU the library runs on holds its own copy of the array from the
 *     first call on that device until the process ends; the first call on a
 *     device looks up the array's address (no allocation call is made,
 *     then or ever).
 *   - Problems whose gdn_chunk_fwd_workspace exceeds the array are refused
 *     with GDN_ERR_SCRATCH before anything is enqueued (B=1, T=4096, H=16,
 *     d=128, bf16 needs 89.25 MiB; B=8, T=2048, H=8 needs 153.5 MiB).
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind; nothing in it needs to start at any value.  Calls that overlap
 *     in time on one GPU (several streams, several host threads) race on
 *     the array and give undefined results: serialise them.
 * Arguments, layouts and the other errors as gdn_chunk_fwd; `stream`
 * decides the device. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_problem* p, const void* q, const void* k,
                                 const void* v, const void* beta,
                                 const void* log_alpha, const float* s0, void* o,
                                 float* s_final, void* stream);

/* The forward with q and k normalised inside ("Gated Delta Networks:
 * Improving Mamba2 with Delta Rule", "Method": the block design passes q and
 * k through an L2 normalisation per token and head; v is left as it is).
 * Computes gdn_chunk_fwd on q_t / |q_t| and k_t / |k_t| (norms over dk, in
 * fp32, per token and head; an all-zero row stays zero).  With the scalar
 * gate or no gate nothing normalised is written: k rows are normalised as
 * the chunk is staged, the q factor is applied to the fp32 products.  With
 * the per-channel gate a prologue pass first writes the normalised q and k
 * rows (input dtype) into the workspace.  Workspace:
 * gdn_chunk_fwd_qknorm_workspace (equal to gdn_chunk_fwd_workspace for the
 * scalar gate and no gate).  Arguments, layouts and errors as
 * gdn_chunk_fwd. */
gdn_status gdn_chunk_fwd_qknorm_workspace(const gdn_problem* p, size_t* bytes);
gdn_status gdn_chunk_fwd_qknorm(const gdn_problem* p, const void* q, const void* k,
                                const void* v, const void* beta,
                                const void* log_alpha, const float* s0, void* o,
                                float* s_final, void* ws, size_t ws_bytes,
                                void* stream);

/* The forward behind the block's q, k, v paths ("Gated Delta Networks:
 * Improving Mamba2 with Delta Rule", "Method": q and k pass through a short
 * convolution, SiLU and an L2 normalisation, v through the same without the
 * normalisation).  The caller's projections xq, xk, xv go through
 *   y[t, h, c] = silu(sum_{j < width} taps[h, c, j] x[t - j, h, c])
 * (causal and depthwise; tap j weighs the input j tokens back; no history
 * before a sequence's first token, so packed sequences never see each
 * other; no bias), q and k rows are then L2-normalised, and gdn_chunk_fwd
 * runs on the results.  With the scalar gate or no gate the k and v rows are
 * convolved (and k normalised) as the forward stages each chunk, and only q
 * goes through a prologue pass that writes it into the workspace in the
 * input dtype; with the per-channel gate the prologue pass writes all three.
 *   width       : taps per channel, 1 .. 8 (else GDN_ERR_UNSUPPORTED).
 *   xq, xk      : [B, T, H, dk] io_dtype;  xv : [B, T, H, dv] io_dtype.
 *   wq, wk      : [H, dk, width] fp32;     wv : [H, dv, width] fp32.
 *   beta, log_alpha, s0, o, s_final : as in gdn_chunk_fwd (every gate).
 *   ws          : at least gdn_chunk_fwd_conv_workspace bytes.
 * Errors as gdn_chunk_fwd. */
gdn_status gdn_chunk_fwd_conv_workspace(const gdn_problem* p, int32_t width, size_t* bytes);
gdn_status gdn_chunk_fwd_conv(const gdn_problem* p, int32_t width, const void* xq,
                              const void* xk, const void* xv, const float* wq,
                              const float* wk, const float* wv, const void* beta,
                              const void* log_alpha, const float* s0, void* o,
                              float* s_final, void* ws, size_t ws_bytes, void* stream);

/* One projection's prologue on its own (the step gdn_chunk_fwd_conv applies
 * to each of q, k, v; "Gated Delta Networks: Improving Mamba2 with Delta
 * Rule", "Method"):  y = silu(conv(x)) with the causal depthwise convolution
 * above, then y / |y| per (token, head) when normalize is non-zero.
 *   d           : the channels of x and y, the problem's dk or dv (else
 *                 GDN_ERR_SHAPE); with normalize, d in {16, 32, 64, 128}.
 *   width       : 1 .. 8 (else GDN_ERR_UNSUPPORTED).
 *   x, y        : [B, T, H, d] io_dtype (packed sequences as in the chunked
 *                 calls, no history across a sequence start).
 *   taps        : [H, d, width] fp32.
 * Only B, T, H, dk, dv, io_dtype, nseq and cu_seqlens of the problem are
 * used (its other fields must still be valid).  Errors as gdn_chunk_fwd. */
gdn_status gdn_prologue_fwd(const gdn_problem* p, int32_t d, int32_t width, int32_t normalize,
                            const void* x, const float* taps, void* y, void* stream);

/* Backward of gdn_prologue_fwd: given dy = dL/dy, writes dx = dL/dx
 * ([B, T, H, d] io_dtype) and dtaps = dL/dtaps ([H, d, width] fp32,
 * overwritten).  The pages define the forward path only; this is its chain
 * rule (the normalisation's projection, SiLU's derivative, the transposed
 * convolution).  The tap gradient sums over every token in a fixed order
 * (deterministic; no atomics).  Workspace: gdn_prologue_bwd_workspace bytes
 * (the fp32 gradient before SiLU and per-block tap partials).  Errors as
 * gdn_chunk_fwd; GDN_ERR_NULL for a NULL dtaps. */
gdn_status gdn_prologue_bwd_workspace(const gdn_problem* p, int32_t d, int32_t width,
                                      size_t* bytes);
gdn_status gdn_prologue_bwd(const gdn_problem* p, int32_t d, int32_t width, int32_t normalize,
                            const void* x, const float* taps, const void* dy, void* dx,
                            float* dtaps, void* ws, size_t ws_bytes, void* stream);

/* Householder-product transitions (the GDN review's "Future work" and its
 * closing section name products of Householder matrices as a way to graft
 * stronger state tracking onto the gated delta rule).  Each token carries
 * nh (key, value, beta) triples; the state is decayed once by the token's
 * alpha and then takes the nh delta-rule steps in order, and the output is
 * read after the last step:
 *   S_t = S_{t-1} alpha_t H_t1 ... H_tnh + writes,  H_tj = I - beta_tj k_tj k_tj^T.
 * The chunked forward runs over the nh * T steps (chunk counts steps).
 *   nh        : 1, 2 or 4 (1 is gdn_chunk_fwd itself).
 *   k, v      : [B, T, nh, H, dk] and [B, T, nh, H, dv] in io_dtype.
 *   beta      : [B, T, nh, H] in gate_dtype.
 *   q         : [B, T, H, dk]; log_alpha [B, T, H] (scalar gate) or NULL
 *               (gate none); the per-channel gate is GDN_ERR_UNSUPPORTED.
 *   o         : [B, T, H, dv]; s0 / s_final as in gdn_chunk_fwd.
 *   p->T and cu_seqlens count tokens, not steps.
 * Errors: GDN_ERR_UNSUPPORTED for another nh or the per-channel gate, the
 * rest as gdn_chunk_fwd. */
gdn_status gdn_chunk_fwd_product_workspace(const gdn_problem* p, int32_t nh,
                                           size_t* bytes);
gdn_status gdn_chunk_fwd_product(const gdn_problem* p, int32_t nh, const void* q,
                                 const void* k, const void* v, const void* beta,
                                 const void* log_alpha, const float* s0, void* o,
                                 float* s_final, void* ws, size_t ws_bytes,
                                 void* stream);

/* Gated DeltaNet-2 with decoupled erase and write strengths.  "Linear
 * Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
 * Routing" (abstract, and its related-paper entry "Gated DeltaNet-2:
 * Decoupling Erase and Write in Linear Attention") names the method and its
 * separate erase and write control but prints no formula.  Reading taken:
 * the single strength beta_t of the gated delta rule splits into an erase
 * strength e_t and a write strength w_t,
 *     S_t = S_{t-1} D_t (I - e_t k_t k_t^T) + w_t v_t k_t^T,
 * with D_t the scalar or per-channel gate as in gdn_chunk_fwd; e = w gives
 * gdn_chunk_fwd, e = 0 gated linear attention.  (In the chunk form e scales
 * the rows of A and W, w those of U.)
 *   erase, write : [B, T, H] in gate_dtype, used as given (never clamped).
 * Everything else (problem, layouts, workspace = gdn_chunk_fwd_workspace,
 * errors) as gdn_chunk_fwd. */
gdn_status gdn2_chunk_fwd(const gdn_problem* p, const void* q, const void* k,
                          const void* v, const void* erase, const void* write,
                          const void* log_alpha, const float* s0, void* o,
                          float* s_final, void* ws, size_t ws_bytes, void* stream);

/* One decode step of the same rule, state in place: Mt = a (.) M,
 * e = w v - e_t Mt^T k, M <- Mt + k e^T, o = M^T q.  erase, write [N, H];
 * the rest as gdn_decode_step. */
gdn_status gdn2_decode_step(const gdn_problem* p, const void* q, const void* k,
                            const void* v, const void* erase, const void* write,
                            const void* log_alpha, float* state, void* o, void* stream);

/* Draft-tree verification for speculative decoding ("TreeWY: Speculative
 * Verification for Gated DeltaNet Hybrids": the gated delta rule as a
 * tree-structured WY transform, every draft node verified by one triangular
 * solve, only the accepted state rebuilt on commit).  Each tree hangs off a
 * committed state; node i carries one token and continues the state of its
 * parent (parent[i] in [-1, i), -1 = the committed state) with one step of
 * the recurrence, and o_i is read from the node's state.  No per-node state
 * is stored: one chunk per tree runs the chunk form with "earlier token"
 * replaced by "ancestor" (path-summed log gates, A and QK^T kept on
 * ancestors only).
 *   p        : B trees of T nodes (dense) or nseq trees packed by
 *              cu_seqlens (B == 1); every tree has at most `chunk` nodes
 *              (dense: T <= chunk, else GDN_ERR_SHAPE; varlen: the caller's
 *              promise, nodes past the chunk get unspecified outputs);
 *              gate none or scalar (per-channel: GDN_ERR_UNSUPPORTED).
 *   parent   : device int32, [B, T] or [total nodes], indices inside each
 *              tree; entries outside [-1, i) are read as -1.
 *   q, k, v, beta, log_alpha : per node, layouts as in gdn_chunk_fwd.
 *   state    : committed states [ntrees, H, dk, dv] fp32 (read only), or
 *              NULL for zeros.
 *   o        : [B, T, H, dv] in io_dtype.
 *   ws       : at least gdn_tree_verify_workspace bytes.
 * Errors as gdn_chunk_fwd, plus GDN_ERR_NULL for a NULL parent. */
gdn_status gdn_tree_verify_workspace(const gdn_problem* p, size_t* bytes);
gdn_status gdn_tree_verify(const gdn_problem* p, const int32_t* parent, const void* q,
                           const void* k, const void* v, const void* beta,
                           const void* log_alpha, const float* state, void* o,
                           void* ws, size_t ws_bytes, void* stream);

/* Commit after a verification: state[m] becomes the state of node
 * accepted[m] of tree m, rebuilt from the committed state along that node's
 * root path (in place; one read and one write of the state).  accepted[m] =
 * -1, or any index outside [0, min(tree size, 64)), leaves state[m] as it is.
 *   p, parent, k, v, beta, log_alpha : as in gdn_tree_verify (q is not
 *              needed); trees of up to 64 nodes.
 *   accepted : device int32 [ntrees].
 *   state    : [ntrees, H, dk, dv] fp32, in/out. */
gdn_status gdn_tree_commit(const gdn_problem* p, const int32_t* parent,
                           const int32_t* accepted, const void* k, const void* v,
                           const void* beta, const void* log_alpha, float* state,
                           void* stream);

/* Workspace bytes gdn_chunk_bwd needs (see gdn_chunk_fwd_workspace). */
gdn_status gdn_chunk_bwd_workspace(const gdn_problem* p, size_t* bytes);

/* Chunkwise backward: gradients of L = <dO, o> + <ds_final, S_final>, the
 * forward recomputed inside (the pages give no backward; this is the
 * adjoint of the recurrence above).  Gradients are taken with respect to
 * log alpha (not alpha) and beta (not a logit).
 *   d_o      : [B, T, H, dv] io_dtype.   ds_final : fp32 or NULL (zeros).
 *   dq, dk   : [B, T, H, dk] io_dtype.   dv : [B, T, H, dv] io_dtype.
 *   dbeta    : [B, T, H] fp32.
 *   dlog_alpha : fp32, shaped like log_alpha; NULL allowed for GATE_NONE.
 *   ds0      : [nseq, H, dk, dv] fp32 or NULL to skip.
 * The result is deterministic (no floating-point atomics).
 * Supported set: as gdn_chunk_fwd.  For fp32 inputs (io_dtype GDN_F32) with
 * the per-channel gate at dk = 128 and chunk = 64 the gradient kernel's LDS
 * plan (fp32 rows and per-channel decays of a 64 x 128 chunk) does not fit
 * in 160 KiB, so that case runs on 32-token chunks (a positive seg_chunks
 * is doubled to keep its length in tokens): the gradients are the same
 * function of the inputs, rounded in another order, and the workspace query
 * returns that plan's size. */
gdn_status gdn_chunk_bwd(const gdn_problem* p, const void* q, const void* k,
                         const void* v, const void* beta,
                         const void* log_alpha, const float* s0,
                         const void* d_o, const float* ds_final, void* dq,
                         void* dk, void* dv, float* dbeta, float* dlog_alpha,
                         float* ds0, void* ws, size_t ws_bytes, void* stream);

/* One token per sequence (B = N sequences), state updated in place:
 *   Mt = a (.) M (a = exp(log alpha), per row for the channel gate),
 *   e = beta (v - Mt^T k),  M <- Mt + k e^T,  o = M^T q.
 * Each state element is read once and written once.
 *   q, k  [N, H, dk]; v [N, H, dv]; beta [N, H]; log_alpha [N, H] or
 *   [N, H, dk]; state [N, H, dk, dv] fp32 in/out; o [N, H, dv] io_dtype. */
gdn_status gdn_decode_step(const gdn_problem* p, const void* q, const void* k,
                           const void* v, const void* beta,
                           const void* log_alpha, float* state, void* o,
                           void* stream);

/* Decode step with Householder-product transitions (the serving side of
 * gdn_chunk_fwd_product; same reading of the GDN review's "Future work"):
 * per (sequence, head) the state is decayed once by alpha, takes the nh
 * delta-rule steps of the token in order, and o = S q is read after the
 * last one; the state is updated in place.
 *   nh        : 1, 2 or 4 (else GDN_ERR_UNSUPPORTED).
 *   q [N, H, dk]; k [N, nh, H, dk]; v [N, nh, H, dv]; beta [N, nh, H];
 *   log_alpha [N, H] (scalar gate) or NULL (gate none); the per-channel
 *   gate is GDN_ERR_UNSUPPORTED.  state [N, H, dk, dv] fp32 in/out;
 *   o [N, H, dv] in io_dtype.  p->B = N; T, chunk and varlen fields are
 *   ignored. */
gdn_status gdn_decode_step_product(const gdn_problem* p, int32_t nh, const void* q,
                                   const void* k, const void* v, const void* beta,
                                   const void* log_alpha, float* state, void* o,
                                   void* stream);

/* Stage timing, for benchmarks and profiling.  While enabled, every kernel
 * the library enqueues is bracketed by a pair of HIP events recorded on the
 * same stream.  gdn_profile_read waits for the recorded events, writes the
 * summed device time (milliseconds) and the number of launches of each stage
 * into total_ms[GDN_STAGE_COUNT] and count[GDN_STAGE_COUNT], and clears the
 * record.  Not for use while a stream is being captured into a graph.
 * Calls that overlap on several host threads are recorded together. */
#define GDN_STAGE_COUNT 12
typedef enum {
  GDN_STAGE_CHUNK_MAP = 0,  /* varlen chunk table                         */
  GDN_STAGE_FWD_PREP = 1,   /* per-chunk gate, UT transform, W/U/P        */
  GDN_STAGE_FWD_SCAN = 2,   /* state recurrence and outputs per segment   */
  GDN_STAGE_DECODE = 3,     /* single-token step                          */
  GDN_STAGE_BWD_STATES = 4, /* backward: chunk-start states               */
  GDN_STAGE_BWD_SCAN = 5,   /* backward: reverse state-gradient pass      */
  GDN_STAGE_BWD_GRAD = 6,   /* backward: per-chunk gradients              */
  GDN_STAGE_OTHER = 7,
  GDN_STAGE_FWD_TRANS = 8,  /* forward: per-segment state maps [M0 | Phi] */
  GDN_STAGE_FWD_COMBINE = 9, /* forward: states entering each segment     */
  GDN_STAGE_TREE_COMMIT = 10, /* draft trees: accepted state rebuilt      */
  GDN_STAGE_PROLOGUE = 11   /* q, k, v paths: convolution, SiLU, L2 norm  */
} gdn_stage;
void gdn_profile_enable(int enable);
gdn_status gdn_profile_read(double* total_ms, int32_t* count);

/* Test hook: when set to a non-zero value every entry point returns
 * GDN_ERR_HIP after validation instead of launching (exercises the launch
 * failure path on machines without a GPU).  Not for production use. */
void gdn_test_set_fail_launch(int enable);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
