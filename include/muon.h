/*
 * libmuon -- the Muon optimizer step's hot path on AMD Instinct MI355X (gfx950).
 *
 * The step, per whole 2D weight matrix (blog "Muon Optimizer + FSDP",
 * section "Background: the conflict between FSDP and Muon"), in three calls:
 *   - refresh the momentum from the gradient   -> muon_momentum_update
 *                                                 (_sq: also the sums of
 *                                                 squares for the norms)
 *   - orthogonalise it by Newton-Schulz        -> muon_newton_schulz_batched
 *   - move the weight by -lr times the result  -> muon_apply
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers to memory the caller owns and
 *     keeps alive until the work enqueued on `stream` has finished.  Matrices
 *     are dense row-major (rows x cols, leading dimension = cols).
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream of the context's device).  Every call only enqueues work; none
 *     synchronises the device, none allocates device memory.
 *   - Arguments are validated before anything is enqueued: on any status
 *     other than MUON_OK nothing was launched.  Faults inside kernels surface
 *     at the caller's next synchronisation, as for any HIP kernel.
 *   - No C++ exception crosses this boundary.
 *   - A context is not thread-safe; use one context per stream (calls made
 *     on different streams with one context must be ordered by the caller).
 */
#ifndef LIBMUON_MUON_H
#define LIBMUON_MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUON_OK = 0,
  MUON_EINVAL = 1,      /* null pointer, bad count/size, aliasing, bad parameter */
  MUON_ESHAPE = 2,      /* rows/cols <= 0, rows % head_rows != 0, ...           */
  MUON_EDTYPE = 3,      /* dtype or dtype combination not supported             */
  MUON_EWORKSPACE = 4,  /* the call needs more workspace than the context holds */
  MUON_EHIP = 5,        /* a HIP runtime call failed (see muon_last_error)      */
  MUON_ENOMEM = 6       /* host-side allocation failed                          */
} muon_status_t;

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype_t;

/* Elements per sum-of-squares partial (muon_momentum_update_sq). */
#define MUON_SQ_BLOCK 4096

/* How the iteration is evaluated (the DeepSpeed PR "[Muon] CPU offload: pin
 * the momentum and overlap the host writeback", section Tests, and the RFC's
 * section 5 Roadmap name an ns_method option with a "gram" choice beside the
 * standard one; neither page spells gram out).
 *   MUON_NS_QUINTIC: the iteration below on the m x n iterate, step by step.
 *   MUON_NS_GRAM:    the same polynomial map carried on m x m matrices only.
 *     With A_0 = X_0 X_0^T and P_k = a I + b A_k + c A_k^2 (a polynomial in
 *     A_k, so symmetric and commuting with it), X_{k+1} = P_k X_k gives
 *     A_{k+1} = P_k A_k P_k and X_steps = (P_{steps-1} ... P_0) X_0.  The
 *     m x n matrix is read twice (A_0 and the final product) instead of three
 *     times per step; every other product is m x m.  The result equals the
 *     quintic's in exact arithmetic; bf16 rounding differs.  A_0 carries the
 *     squared singular values, which bf16 resolves only when the matrix is
 *     far from square: in BF16 compute the Gram form runs on units with
 *     2 m <= n and the quintic iteration on the others (F32: always). */
typedef enum { MUON_NS_QUINTIC = 0, MUON_NS_GRAM = 1 } muon_ns_method_t;

/* Whole-iteration fusion for small units: a wide BF16 unit with m <= 128
 * (e.g. the 128 x n heads of per-head Muon, RFC section 4D) can run every
 * iteration in one launch, one workgroup per unit holding A and B (and, for
 * MUON_NS_GRAM, the m x m iterates) in on-chip memory.  The quintic
 * accumulates the next iteration's Gram product while the update is stored,
 * so the iterate is read once and written once per iteration; the Gram form
 * reads the input twice and writes the result once in all.  Results are
 * bit-identical to the unfused kernels.  AUTO fuses when the call has at
 * least as many units as the device has compute units (every CU gets a
 * unit), or when n <= 3072 (a workgroup then finishes its unit before the
 * separate launches would, however many CUs stay idle); ON whenever
 * eligible; OFF never.  Not eligible: tall units, m < 16 (those run in
 * fp32, see muon_newton_schulz_batched), m > 128, F32 compute, a
 * per-iteration coefficient table of more than
 * MUON_NS_FUSED_MAX_ROWS rows, and outputs that overlap an input other than
 * their own (in place, unit for unit, is fine). */
typedef enum { MUON_FUSE_AUTO = 0, MUON_FUSE_OFF = 1, MUON_FUSE_ON = 2 } muon_fuse_t;
#define MUON_NS_FUSED_MAX_ROWS 16

/* Newton-Schulz parameters.  The quintic iteration is the one the DeepSpeed
 * RFC "Enable Correct and High-Performance Muon Optimizer under ZeRO CPU
 * Offload" calls the current default (section 5, Roadmap), run for five to
 * six iterations (section 2, Root Cause Analysis).  Per iteration, on the
 * normalised matrix X (m x n, m <= n):
 *     A = X X^T ;  B = b A + c A A ;  X <- a X + B X
 * (the library forms B' = a I + B and computes X <- B' X, the same product
 * with one operand fewer).
 * X_0 = Y / (||Y||_F + eps); a tall Y (rows > cols) is processed as Y^T and
 * the result transposed back.  Defaults (muon_ns_params_default):
 * steps 5, (a, b, c) = (3.4445, -4.7750, 2.0315), eps 1e-7, compute BF16,
 * coeffs NULL.
 * Per-iteration coefficients (RFC section 5, Roadmap: coefficients optimised
 * for each iteration, "Polar Express"): when coeffs is not NULL it points to
 * `steps` rows of three floats (a_k, b_k, c_k), row-major, in HOST memory,
 * read during the call only; iteration k uses row k in place of (a, b, c)
 * (Gram form: P_k = a_k I + b_k A_k + c_k A_k^2).  Every value must be
 * finite.  muon_ns_minimax_coeffs fills such a table. */
typedef struct {
  int32_t steps;     /* >= 0 */
  float a, b, c;     /* quintic coefficients */
  float eps;         /* added to the Frobenius norm, >= 0 */
  int32_t compute;   /* muon_dtype_t: BF16 = bf16 MFMA with fp32 accumulate,
                        F32 = fp32 verification mode */
  int32_t method;    /* muon_ns_method_t, default MUON_NS_QUINTIC */
  int32_t fuse;      /* muon_fuse_t, default MUON_FUSE_AUTO */
  const float* coeffs; /* NULL, or steps x 3 per-iteration (a, b, c), host */
  /* Norms from the momentum pass (see muon_momentum_update_sq): NULL, or the
   * DEVICE array of sq_count partials that pass wrote for the update buffer
   * starting at the device address sq_base.  Every unit must then begin
   * sq_base + a whole number of MUON_SQ_BLOCK elements and span whole blocks
   * (its elements a multiple of MUON_SQ_BLOCK), inside the sq_count blocks;
   * its norm is the sum of its blocks' partials (fixed order) and the inputs
   * are not read for it.  The partials must describe the current contents of
   * the units (the caller's ordering).  Violations: MUON_EINVAL. */
  const double* sq_partials;
  const void* sq_base;
  int64_t sq_count;
} muon_ns_params_t;

/* Geometry of one weight matrix (RFC section 4A: keep the 2D shape and head
 * dimensions with the parameter).  head_rows = 0: the whole matrix is one
 * Newton-Schulz unit; head_rows = h > 0: rows/h contiguous row blocks of
 * h x cols are orthogonalised independently (RFC section 4D, per-head Muon;
 * blog section "Chunked communication": split fused tensors into their
 * logical matrices, never row-split one matrix). */
typedef struct {
  int64_t rows, cols, head_rows;
} muon_shape_t;

typedef struct muon_ctx muon_ctx_t;
typedef struct muon_plan_s muon_plan_t;

/* ------------------------------------------------------------------------ */
/* Context and workspace                                                     */
/* ------------------------------------------------------------------------ */

/* Create a context on HIP device `device` holding one preallocated device
 * workspace slab of `workspace_bytes` (blog section "Memory control", item 2:
 * preallocate the workspace once and only take views of it per micro-bucket).
 * This is the only call that allocates device memory.  On success *out owns
 * the slab until muon_destroy.  Errors: MUON_EINVAL (out NULL),
 * MUON_EHIP (no such device / allocation failed), MUON_ENOMEM. */
muon_status_t muon_create(int device, size_t workspace_bytes, muon_ctx_t** out);

/* Free the context and its workspace (blog section "Memory control", item 2:
 * the workspace lives as long as the context).  Waits for the context's
 * device to finish the work enqueued so far.  NULL is accepted. */
muon_status_t muon_destroy(muon_ctx_t* ctx);

/* Size of the context's workspace slab in bytes (0 for NULL; blog section
 * "Memory control", item 2). */
size_t muon_ctx_workspace_bytes(const muon_ctx_t* ctx);

/* Fill *p with the defaults listed above (RFC section 5, Roadmap: the
 * quintic iteration is the current default; section 2: five to six
 * iterations). */
void muon_ns_params_default(muon_ns_params_t* p);

/* Per-iteration coefficients (RFC section 5, Roadmap: Newton-Schulz with
 * coefficients optimised per iteration, so that fewer iterations reach the
 * same accuracy; the page gives no table).  Iteration t maps each singular
 * value x to p_t(x) = a x + b x^3 + c x^5, where p_t is the odd quintic with
 * the smallest max |1 - p(x)| over [l_t, u_t (1 + margin)], the interval
 * that holds the singular values at that point; l_0 = lo, u_0 = 1 (X_0 is
 * normalised by its Frobenius norm), and the next interval is p_t's image
 * [1 - E_t, 1 + E_t], E_t the attained maximum.  `margin` widens each
 * interval at the top, where p_t climbs steeply, so that values that bf16
 * rounding pushes slightly past it stay bounded and rounding errors near
 * the top are amplified less (0.05 is the binding's default: a few bf16
 * roundings of 2^-8 each, with room).  An interval narrower than 1e-3 takes the limit
 * polynomial (15/8, -5/4, 3/8).  Pure host function, computed in double.
 * out: `steps` x 3 floats (caller-owned, host).  *bound (may be NULL)
 * receives E_{steps-1}: in exact arithmetic every singular value of X_0 in
 * [lo, 1] ends within [1 - bound, 1 + bound].  `margin` must lie in [0.01, 0.1]:
 * with bf16 iterates, low-rank inputs reached relative errors of 0.36 at
 * margin 0 and 0.14 at margin 0.2 against the fp64 iteration with the same
 * coefficients, and stayed within 2e-2 inside that window.  Errors:
 * MUON_EINVAL (steps < 1 or > 1024, lo outside (0, 1), margin outside
 * [0.01, 0.1], out NULL, or the exchange did not converge). */
muon_status_t muon_ns_minimax_coeffs(int32_t steps, double lo, double margin, float* out,
                                     double* bound);

/* Workspace one muon_newton_schulz_batched call needs for `count` matrices
 * of `shape` in compute dtype `compute` (pure host function; blog section
 * "Memory control", item 2).  Per Newton-Schulz unit of m x n (m = min, n =
 * max of its rows and cols, e = element bytes of the compute dtype): two
 * iterate buffers (2 e m n) + A and B (2 e m^2) + 8 bytes of scalars + 8
 * bytes per norm partial (at most 512); in BF16 also the iterate's rounding
 * residual (2 bytes per element, rows and columns padded to the tile: 256
 * once m >= 256, else 128) and B's diagonal in fp32 (4 m).  Each region is
 * rounded up to 256 bytes: (2 + 2 m/n) x the unit's e m n bytes (BF16:
 * 3 + 2 m/n, up to the residual's padding) plus scalars.  BF16 units with
 * m < 16 run the iteration in fp32: for them it is at least the inputs
 * widened to fp32 (4 m n) plus the F32 figure.  Returns 0 for an invalid
 * shape or count <= 0. */
size_t muon_ns_workspace_bytes(muon_shape_t shape, int64_t count, int32_t compute);

/* Workspace to run Newton-Schulz over a list of matrices of mixed shapes,
 * one muon_newton_schulz_batched call per group of identical shapes
 * (rows, cols, head_rows), the calls one after another on one context: the
 * largest group's muon_ns_workspace_bytes (blog section "Memory control",
 * item 2: the workspace is a stated function of what one call holds).  Pure
 * host function.  Returns 0 when count <= 0 or a shape is invalid. */
size_t muon_workspace_bytes(const muon_shape_t* shapes, int64_t count, int32_t compute);

/* ------------------------------------------------------------------------ */
/* Host scheduler: same-shape buckets split into micro-buckets under a cap   */
/* ------------------------------------------------------------------------ */

typedef enum {
  MUON_CAP_FULL_BYTES = 0,  /* sum of full-matrix bytes (e * rows * cols) <= cap */
  MUON_CAP_WORKSPACE = 1    /* sum of Newton-Schulz workspace bytes      <= cap */
} muon_cap_kind_t;

typedef struct {
  int64_t m, n;               /* canonical shape of the bucket's units (m <= n) */
  int64_t count;              /* matrices in this micro-bucket                 */
  int64_t units;              /* Newton-Schulz units (heads expanded)          */
  int64_t numel;              /* elements of its matrices                      */
  size_t full_bytes;          /* e * numel                                      */
  size_t workspace_bytes;     /* sum of muon_ns_workspace_bytes per shape group */
  int32_t over_cap;           /* 1 if a single matrix alone exceeds the cap     */
  int32_t shape_groups;       /* distinct (rows, cols, head_rows) runs inside   */
  int64_t elem_offset;        /* its first element in the plan's flat layout   */
} muon_bucket_info_t;

/* Group `count` matrices into buckets by canonical unit shape (m, n) in order
 * of first appearance (blog section "Memory control", item 6: merge same-shape
 * matrices across layers into one bucket), order each bucket's members by
 * orientation (units of the first member's orientation first: wide units,
 * rows <= cols, and tall ones run separate launches) and then by exact shape
 * (stable), so that members whose units share a shape lie together, and cut
 * each bucket into micro-buckets of whole
 * matrices whose cost stays within `cap_bytes` (blog sections "Chunked
 * communication" and "Memory control", item 1: a separate Muon cap;
 * estimate_muon_peak(bucket) <= cap).  A matrix larger than the cap gets a
 * micro-bucket of its own, flagged over_cap.
 * compute_units = 0: micro-buckets are filled greedily up to the cap.
 * compute_units = C > 0 (the device's CU count): the cut points are chosen,
 * still under the cap, to minimise a model of the Newton-Schulz time on C
 * CUs -- each product launch takes ceil(tiles / slots) rounds of its
 * per-tile k-length (one 256-tile per CU, or two 128-tiles per CU at 0.6 of
 * a 256-tile round where the launch takes those because few 256-tiles would
 * leave most CUs idle), each orientation of a micro-bucket its own
 * launches -- plus a
 * fixed cost per launch chain, so that launches do not end with a nearly
 * empty last round of tiles.  Host only; *out is owned by the
 * caller (muon_plan_destroy).  Errors: MUON_EINVAL, MUON_ESHAPE. */
muon_status_t muon_plan_create(const muon_shape_t* shapes, int64_t count, size_t cap_bytes,
                               int32_t cap_kind, int32_t compute, int32_t compute_units,
                               muon_plan_t** out);
/* muon_plan_create with BF16 compute and the plain cap-filling cuts
 * (compute_units = 0): the scheduler's signature with the cap and its kind
 * only (blog sections "Chunked communication" and "Memory control", items 1
 * and 6). */
muon_status_t muon_plan(const muon_shape_t* shapes, int64_t count, size_t cap_bytes,
                        int32_t cap_kind, muon_plan_t** out);
/* Number of micro-buckets (blog section "Chunked communication"). */
int64_t muon_plan_num_buckets(const muon_plan_t* plan);
/* Info on micro-bucket `b`.  When non-NULL, `indices` receives info->count
 * matrix indices (positions in the `shapes` array) in execution order, and
 * `offsets` the element offset of each of those matrices in the plan's flat
 * layout: state buffers (gradients, momentum, weights) that hold every matrix
 * in plan order -- micro-bucket after micro-bucket, members packed in
 * execution order -- so that each micro-bucket is one contiguous range
 * starting at info->elem_offset (blog section "DBuffer": addresses planned
 * once at init, views per step).  Errors: MUON_EINVAL (NULL plan or info, b
 * out of range). */
muon_status_t muon_plan_bucket(const muon_plan_t* plan, int64_t b, muon_bucket_info_t* info,
                               int64_t* indices, int64_t* offsets);
/* Elements of the plan's flat layout (the sum of every matrix's rows x cols;
 * blog section "DBuffer": one persistent buffer per state). */
int64_t muon_plan_total_elems(const muon_plan_t* plan);
/* Largest workspace_bytes over the plan's micro-buckets: a context this large
 * runs every micro-bucket (blog section "Memory control", item 2: one
 * preallocated workspace sized by the cap). */
size_t muon_plan_max_workspace(const muon_plan_t* plan);
/* Free a plan (NULL is accepted; blog section "Memory control": the plan is
 * made once at init and kept). */
void muon_plan_destroy(muon_plan_t* plan);

/* ------------------------------------------------------------------------ */
/* The three steps                                                           */
/* ------------------------------------------------------------------------ */

/* Momentum with Nesterov look-ahead over `numel` contiguous elements
 * (blog, section "Background": the momentum refresh; RFC section 2:
 * the first-order momentum the offload path must keep).  Per element, each
 * operation one IEEE binary32 rounding, no fused multiply-add:
 *     t  = (1 - beta) * g
 *     M' = beta * M + t                      (written back to momentum)
 *     U  = t + beta * M'   (nesterov != 0)   or   U = M'   (nesterov == 0)
 * grad: `grad_dtype` (BF16 or F32); momentum: F32, updated in place;
 * update_out: `update_dtype` (BF16 = U rounded to nearest-even, or F32).
 * numel == 0 is a no-op.  update_out may not alias grad or momentum; all
 * pointers must be element-aligned.  Errors: MUON_EINVAL (NULL pointer,
 * numel < 0, aliasing, beta outside [0, 1]), MUON_EDTYPE, MUON_EHIP. */
muon_status_t muon_momentum_update(muon_ctx_t* ctx, void* stream, const void* grad,
                                   int32_t grad_dtype, float* momentum, void* update_out,
                                   int32_t update_dtype, int64_t numel, float beta,
                                   int32_t nesterov);

/* muon_momentum_update, which also leaves the sums of squares that the
 * Newton-Schulz normalisation X_0 = U / (||U||_F + eps) needs (blog section
 * "Background": Newton-Schulz runs on the refreshed momentum; the sums of
 * squares come out of the same pass, so the Frobenius norms need no second
 * read of U).  sq_partials (device,
 * ceil(numel / MUON_SQ_BLOCK) doubles, caller-owned) receives for block b the
 * sum of squares of update elements [b*4096, min((b+1)*4096, numel)) as
 * stored (bf16 values when update_dtype is BF16), in binary64: every square
 * is exact, the sum runs in a fixed order, so the partials are reproducible
 * bit for bit.  Pass them to muon_newton_schulz_batched through
 * muon_ns_params_t.sq_partials.  Errors: those of muon_momentum_update, and
 * MUON_EINVAL for a NULL or overlapping sq_partials. */
muon_status_t muon_momentum_update_sq(muon_ctx_t* ctx, void* stream, const void* grad,
                                      int32_t grad_dtype, float* momentum, void* update_out,
                                      int32_t update_dtype, int64_t numel, float beta,
                                      int32_t nesterov, double* sq_partials);

/* Batched Newton-Schulz over one same-shape group (blog section "Chunked
 * communication": every Muon unit stays a whole matrix; XTuner-style same-
 * shape buckets).  mats: HOST array of `count` device pointers to rows x cols
 * matrices of io_dtype; out: HOST array of `count` device pointers receiving
 * the orthogonalised update in the same shape and dtype (out == NULL, or
 * out[i] == mats[i], means in place).  With shape.head_rows = h > 0 every
 * h x cols row block is orthogonalised on its own.  Supported (io_dtype,
 * params->compute): (BF16, BF16) -- bf16 MFMA, fp32 accumulate, A, B and
 * the X iterates rounded to bf16 (units whose smaller side is under 16:
 * the iteration in fp32 on widened inputs, the result rounded to bf16);
 * (F32, F32) -- fp32 verification mode.
 * The Frobenius norm is reduced deterministically (fixed order), so two
 * calls on identical inputs give identical bits.  A unit whose norm is 0
 * yields exactly 0.  nonfinite_flag (device int, may be NULL) gets 1 OR-ed
 * in when some unit's norm is not finite; values are propagated, never
 * skipped.  Uses the context workspace (muon_ns_workspace_bytes(shape,
 * count, compute) bytes).  count == 0 is a no-op.  The call may be recorded
 * into a HIP graph (stream capture) when the inputs, and the outputs, are
 * evenly spaced; irregularly placed matrices need pointer tables uploaded
 * from a host ring that later calls reuse, and are rejected while the
 * stream captures (MUON_EINVAL).  Errors: MUON_EINVAL, MUON_ESHAPE,
 * MUON_EDTYPE, MUON_EWORKSPACE, MUON_EHIP. */
muon_status_t muon_newton_schulz_batched(muon_ctx_t* ctx, void* stream, const void* const* mats,
                                         int64_t count, muon_shape_t shape, int32_t io_dtype,
                                         const muon_ns_params_t* params, void* const* out,
                                         int* nonfinite_flag);

/* Weight apply over `numel` contiguous elements (blog, section "Background":
 * the weight moves by -lr times the orthogonalised update).  Each
 * operation one binary32 rounding, no FMA:
 *     eta = lr * scale;  W1 = W * (1 - lr * weight_decay) if weight_decay != 0
 *     W'  = W1 - eta * u                        (written back to master)
 *     weight_bf16 = W' rounded to nearest-even  (when weight_bf16 != NULL)
 * update: `update_dtype` (BF16 or F32).  numel == 0 is a no-op.
 * Errors: MUON_EINVAL (NULL master/update, numel < 0, aliasing),
 * MUON_EDTYPE, MUON_EHIP. */
muon_status_t muon_apply(muon_ctx_t* ctx, void* stream, float* master, const void* update,
                         int32_t update_dtype, void* weight_bf16, int64_t numel, float lr,
                         float scale, float weight_decay);

/* Allocation-free Newton-Schulz, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and results as
 * muon_newton_schulz_batched (bit for bit), without a context: the workspace
 * is a static device array of MUON_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds from the first call there until the process ends
 * (the first call on a device looks its address up; no call allocates).
 * device: the HIP device the stream belongs to.  The call's workspace
 * (muon_ns_workspace_bytes(shape, count, params->compute)) must fit the
 * scratch, else MUON_EWORKSPACE.  Matrices must be evenly spaced (mats[i] =
 * mats[0] + i * d, no overlap), and out NULL (in place), equal to mats, or
 * evenly spaced and disjoint from every input; otherwise MUON_EINVAL.  Every
 * call on one GPU shares that GPU's scratch: calls that overlap on one GPU
 * (different streams or threads, without ordering) race and give undefined
 * results.  No per-kernel timing.  muon_noalloc_last_error() gives the
 * calling thread's last error text (a static string). */
#define MUON_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
muon_status_t muon_newton_schulz_batched_noalloc(int device, void* stream,
                                                 const void* const* mats, int64_t count,
                                                 muon_shape_t shape, int32_t io_dtype,
                                                 const muon_ns_params_t* params,
                                                 void* const* out, int* nonfinite_flag);
const char* muon_noalloc_last_error(void);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                               */
/* ------------------------------------------------------------------------ */

/* Static text for a status code ("unknown status" for values outside the
 * enum).  Error reporting is part of the per-bucket diagnostics the blog's
 * section "Metrics to record" asks for. */
const char* muon_status_string(muon_status_t s);
/* Text of the last error recorded on ctx (empty string when none; NULL ctx
 * gives a static text), blog section "Metrics to record". */
const char* muon_last_error(const muon_ctx_t* ctx);

/* Per-kernel-class timing with HIP events recorded on the launch stream
 * around each kernel (per-bucket timing, blog section "Metrics to record").
 * enable != 0 preallocates an event pool; launches beyond its capacity, and
 * launches recorded into a graph (stream capture), are not timed.  muon_timing_read synchronises on the recorded events and
 * returns the summed duration and number of timed launches of one class. */
typedef enum {
  MUON_K_MOMENTUM = 0,
  MUON_K_NORM = 1,
  MUON_K_GRAM = 2,
  MUON_K_SYMSQ = 3,
  MUON_K_UPDATE = 4,
  MUON_K_APPLY = 5,
  MUON_K_PROD = 6,   /* m x m products of MUON_NS_GRAM (P_k Q_k, P_k A_k, (P_k A_k) P_k) */
  MUON_K_FUSED = 7,  /* whole-iteration launches of small units (muon_fuse_t) */
  MUON_K_COUNT = 8
} muon_kernel_class_t;

muon_status_t muon_timing_enable(muon_ctx_t* ctx, int32_t enable, int32_t capacity);
/* Time only the kernel classes whose bit (1u << muon_kernel_class_t) is set
 * in class_mask: launches of the other classes record no events, and so
 * add no event markers to their stream (every class is timed by default;
 * 0 times none).  Takes effect for launches enqueued after the call.
 * Errors: MUON_EINVAL (ctx NULL, or a bit at or above MUON_K_COUNT set). */
muon_status_t muon_timing_select(muon_ctx_t* ctx, uint32_t class_mask);
muon_status_t muon_timing_reset(muon_ctx_t* ctx);
muon_status_t muon_timing_read(muon_ctx_t* ctx, int32_t kernel_class, double* total_ms,
                               int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* LIBMUON_MUON_H */
