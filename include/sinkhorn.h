/*
 * sinkhorn.h -- C ABI of the MI355X (gfx950) log-domain Sinkhorn half-step library.
 *
 * The method (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
 * section "Metodologia", part "1. Riformulazione in Forma di Attenzione", Proposizione 1): for
 * squared-Euclidean cost
 * C_ij = ||x_i - y_j||^2 the stabilised log-domain update
 *
 *     f_i <- -eps * LSE_j [ (g_j - C_ij)/eps + log b_j ]
 *
 * equals ||x_i||^2 - eps * LSE_j [ (2 x_i.y_j + g_j - ||y_j||^2 + eps log b_j) / eps ],
 * i.e. the row log-sum-exp of a dot-product score matrix plus a per-column bias.
 * The g update is the same operation with the two clouds exchanged.  Each half-step
 * runs as one streaming pass (part "2. Kernel di Streaming e Tassellazione" of the
 * same section: no n x m matrix in HBM, online max / sum-exp, row-stationary traversal).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Problem shape (sk_problem): `batch` independent problems, each with n source
 *    points X[b] (n x d) and m target points Y[b] (m x d), row-major, contiguous:
 *    X is [batch][n][d], Y is [batch][m][d], element type `dtype` (fp32 or bf16).
 *    Weights a [batch][n], b [batch][m] and potentials f [batch][n], g [batch][m]
 *    are fp32.  All of these are DEVICE pointers owned by the caller.
 *  - Weights must be positive and each row must have at least one positive
 *    weight; a zero weight removes that point (its log is -inf).  Weights need not
 *    sum to one (the update is exact for any positive weights).
 *  - ws / ws_bytes: a caller-owned DEVICE workspace of at least
 *    sinkhorn_workspace_bytes(p) bytes.  The library never allocates device or
 *    pinned memory and keeps no state between calls other than what it writes
 *    into ws.  sinkhorn_init_norms must have run on the same ws (same X, Y, a, b)
 *    before half-steps or the marginal error are called, and must run again
 *    after X, Y, a or b change: ws keeps operand rows derived from them (for fp32
 *    inputs, per-eps key rows that later calls at the same eps reuse).
 *  - stream: a HIP stream; every call only enqueues work on it and returns
 *    without synchronising.  The caller synchronises before reading outputs.
 *    Concurrent calls that share one ws race.
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    on failure nothing is launched, a status code is returned and
 *    sinkhorn_last_error() describes it.  A failed launch returns SK_EHIP.
 *    NaN or inf inside the data is not checked and propagates.
 *  - eps: positive and finite.  Log base is natural everywhere in the outputs.
 *  - Centring: the squared-Euclidean cost depends only on x_i - y_j, so
 *    sinkhorn_init_norms moves both clouds of each problem by one common vector c
 *    (the centre of their joint bounding box, computed in fp64 on the device)
 *    before any norm or operand is formed.  f and g are unchanged by this (they
 *    are the potentials of the given points); barycentric projections are
 *    returned in the given coordinates.  bf16 inputs are centred only when every
 *    x - c is itself a bf16 value (clouds far from the origin compared with
 *    their spread); otherwise c = 0.  The cosine cost is never centred.
 *  - Supported score range: with lambda = log2(e)/eps and R the largest
 *    |coordinate - c| of the two clouds (1 under the cosine cost), the base-2
 *    scores lambda*(2 x.y + g_j - |y_j|^2 + eps log b_j) of the centred points
 *    must stay below 2^22 in magnitude, roughly lambda * 6 d R^2 < 4e6 (for
 *    eps = 0.01 and d = 3: R up to a few tens).  Beyond it the lazy row offsets
 *    lose the headroom that keeps the exponentials finite: the kernels then set
 *    SK_FLAG_SCORE_RANGE in the workspace's status word, and outputs may be
 *    inaccurate or non-finite.  Any non-finite potential written sets
 *    SK_FLAG_NONFINITE.  sinkhorn_range_flags reads the word; init clears it.
 */
#ifndef SINKHORN_MI355X_H
#define SINKHORN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SK_OK = 0,
    SK_EINVAL = 1,       /* bad argument: NULL pointer, eps <= 0 or non-finite, iters < 0, unknown cost ... */
    SK_ESHAPE = 2,       /* batch, n, m or d out of range */
    SK_EDTYPE = 3,       /* unknown dtype */
    SK_EHIP = 4,         /* a HIP launch or runtime call failed */
    SK_EUNSUPPORTED = 5, /* valid but not supported by this build (d too large) */
    SK_EWORKSPACE = 6    /* workspace missing or smaller than sinkhorn_workspace_bytes */
} sk_status;

typedef enum { SK_FP32 = 0, SK_BF16 = 1 } sk_dtype; /* element type of X and Y */

/* Bits of the workspace's status word (an OR over every call since the last
 * sinkhorn_init_norms on that workspace). */
#define SK_FLAG_SCORE_RANGE 1u /* a score beyond the supported range (see above) */
#define SK_FLAG_NONFINITE 2u   /* a potential written as NaN or +-inf */

/* Size of the built-in scratch array of sinkhorn_solve_noalloc (bytes). */
#define SK_NOALLOC_MAX_BYTES (64u * 1024u * 1024u)

/* Largest supported point dimension (the pages' largest, section "Risultati
 * Sperimentali": d up to 1024).  Half-steps, solves and marginal errors: d <=
 * SK_MAX_D for bf16 inputs and d <= SK_MAX_D_FP32 for fp32 inputs.  fp32 inputs
 * with d <= SK_MAX_D_SPLIT take the exact grid/remainder operand layout (seven
 * correction products per coordinate, kept in registers); wider ones a hi/lo
 * layout (three bf16 products per coordinate, 2^-16 relative per product,
 * accumulated in fp32) streamed through LDS with a K loop.  The transport,
 * plan-product and HVP calls take the same d.  Up to SK_MAX_D_TRANSPORT (bf16
 * inputs) or SK_MAX_D_SPLIT (fp32 inputs, cosine cost) their P.V pass keeps the
 * query operand in registers and never stores a weight; wider problems first
 * take the rows' half-step, then write the weights of one block of rows against
 * all keys (bf16 hi/lo parts, at most 1 GiB of the transport workspace) and
 * multiply them with the value rows in a second blocked MFMA pass; fp32
 * coordinates enter that product in two bf16 parts (16 significant bits).
 * Larger d returns SK_EUNSUPPORTED. */
#define SK_MAX_D 1024
#define SK_MAX_D_FP32 1024
#define SK_MAX_D_SPLIT 88
#define SK_MAX_D_TRANSPORT 256

/* Ground cost.  SK_COST_SQEUCLID: C_ij = ||x_i - y_j||^2 (the pages' cost).
 * SK_COST_COSINE: the cosine distance after normalisation (page "FlashSinkhorn: Trasporto Ottimo
 * Entropico Consapevole delle I/O su GPU", section "Significato e Affermazioni"), taken as the
 * squared distance
 * between the normalised points, C_ij = ||x_i/|x_i| - y_j/|y_j|||^2
 * = 2 - 2 cos(x_i, y_j); a zero point stays zero (cost 1 to any other point).
 * The cosine cost runs on the split fp32 layout, so d <= SK_MAX_D_SPLIT for
 * either dtype. */
typedef enum { SK_COST_SQEUCLID = 0, SK_COST_COSINE = 1 } sk_cost;

typedef struct {
    int64_t batch; /* >= 1 independent problems */
    int64_t n;     /* >= 1 source points per problem */
    int64_t m;     /* >= 1 target points per problem */
    int64_t d;     /* 1 .. SK_MAX_D (bf16), SK_MAX_D_FP32 (fp32), SK_MAX_D_SPLIT (cosine cost) */
    int32_t dtype; /* sk_dtype of X and Y */
    int32_t cost;  /* sk_cost; 0 = squared Euclidean */
} sk_problem;

/* Bytes of device workspace needed for problem p (0 if p is invalid; see
 * sinkhorn_last_error).  Linear in batch*(n+m)*d: the n x m matrix is never stored. */
size_t sinkhorn_workspace_bytes(const sk_problem* p);

/* Precompute ||x_i||^2, ||y_j||^2, log a_i, log b_j and the kernels' operand
 * layouts of X and Y into ws (the precomputed log-weight biases of Proposizione 1).
 * X, Y: [batch][n|m][d] of dtype p->dtype; a, b: fp32 weights. */
sk_status sinkhorn_init_norms(const sk_problem* p, const void* X, const void* Y,
                              const float* a, const float* b, void* ws, size_t ws_bytes,
                              void* stream);

/* One f half-step: f_i = -eps * LSE_j[(g_j - C_ij)/eps + log b_j] for every problem.
 * g [batch][m] in, f [batch][n] out (f and g must not overlap).  X and Y are the
 * arrays given to sinkhorn_init_norms. */
sk_status sinkhorn_half_step_f(const sk_problem* p, const void* X, const void* Y, void* ws,
                               size_t ws_bytes, const float* g, float eps, float* f, void* stream);

/* One g half-step: g_j = -eps * LSE_i[(f_i - C_ij)/eps + log a_i]: the f step with
 * the roles of X and Y exchanged, read in the same point-major layout (no transposed
 * copy).  f [batch][n] in, g [batch][m] out. */
sk_status sinkhorn_half_step_g(const sk_problem* p, const void* X, const void* Y, void* ws,
                               size_t ws_bytes, const float* f, float eps, float* g, void* stream);

/* Full solve: init_norms, then `iters` iterations of (f half-step, g half-step): the
 * repeated Sinkhorn iterations of the problem statement (same page, section
 * "Enunciato del Problema": entropic OT solved by Sinkhorn iterations, at scale and
 * repeatedly) with the updates of part "1. Riformulazione in Forma di Attenzione".
 * eps: HOST array of n_eps floats; n_eps == 1 means a constant eps, n_eps == iters
 * means iteration k uses eps[k] for both half-steps (an annealing schedule).
 * f and g are in/out: the f half-step runs first, so only the incoming g matters
 * (pass zeros for a cold start, or a saved g to resume).  iters == 0 only runs
 * init_norms. */
sk_status sinkhorn_solve(const sk_problem* p, const void* X, const void* Y, const float* a,
                         const float* b, const float* eps, int64_t n_eps, int64_t iters,
                         float* f, float* g, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free solve, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): sinkhorn_solve without ws and ws_bytes.  Its workspace is a
 * scratch array built into the library, SK_NOALLOC_MAX_BYTES per GPU, held by
 * every GPU the library runs on until the process ends.  Problems whose
 * sinkhorn_workspace_bytes exceeds that size return SK_EWORKSPACE before
 * anything is enqueued.  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (other streams or threads) race, and the
 * array keeps the last call's contents (each call starts with the set-up of
 * sinkhorn_init_norms, which clears what must start at zero).
 * flags: optional DEVICE word (NULL: not reported) that receives the status
 * word (SK_FLAG_*) of this solve, stream-ordered.  Allocates nothing: no
 * hipMalloc, no hipFree, no allocating library call. */
sk_status sinkhorn_solve_noalloc(const sk_problem* p, const void* X, const void* Y, const float* a,
                                 const float* b, const float* eps, int64_t n_eps, int64_t iters,
                                 float* f, float* g, uint32_t* flags, void* stream);

/* Copy the status word of ws (an OR of SK_FLAG_* over every call since the last
 * sinkhorn_init_norms on ws) into the DEVICE word *flags, stream-ordered (no
 * synchronisation).  A diagnostic of this library, not an operation of the pages. */
sk_status sinkhorn_range_flags(const sk_problem* p, const void* ws, size_t ws_bytes, uint32_t* flags,
                               void* stream);

/* L1 marginal errors of the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps).  Not an
 * operation of the pages: a requested convergence diagnostic of this library's API.
 * err[2*k]   = sum_i | sum_j P_ij - a_i |   (rows of problem k)
 * err[2*k+1] = sum_j | sum_i P_ij - b_j |   (columns of problem k)
 * computed without forming P (row sums are a_i exp((f_i - T_f(g)_i)/eps)).
 * err is a DEVICE array of 2*batch floats.  Uses ws scratch (after init_norms). */
sk_status sinkhorn_marginal_error(const sk_problem* p, const void* X, const void* Y, void* ws,
                                  size_t ws_bytes, const float* f, const float* g, float eps,
                                  float* err, void* stream);

/* ---------------------------------------------------------------------------
 * Transport application (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
 * section "Metodologia", part "3. Differenziazione e Ottimizzazione del Secondo Ordine": the barycentric
 * projection and the gradient are weighted averages over the transport plan,
 * computed by the same streaming pass without forming the plan).
 *
 * For the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) of potentials f, g:
 *   sinkhorn_barycentric_x:  bary_i = sum_j P_ij y_j / sum_j P_ij        [batch][n][d]
 *                            grad_i = sum_j P_ij 2 (x_i - y_j)           [batch][n][d]
 *                                   = 2 r_i (x_i - bary_i),  r_i = sum_j P_ij
 *   sinkhorn_barycentric_y:  the same for the points of Y (columns of P):
 *                            bary_j = sum_i P_ij x_i / sum_i P_ij,
 *                            grad_j = sum_i P_ij 2 (y_j - x_i)            [batch][m][d]
 * grad is the gradient of <P, C> in the points with the plan held fixed, which
 * at converged potentials is the gradient of the entropic OT value (envelope
 * theorem).  bary does not depend on the potential of its own side.
 * Under the cosine cost, bary is the projection among the normalised points of
 * the other cloud, and grad is taken in the raw points (through the
 * normalisation: it is orthogonal to its point).
 * bary and grad are fp32 DEVICE arrays owned by the caller; grad may be NULL.
 * These calls need a workspace of sinkhorn_transport_workspace_bytes(p) (a
 * superset of the solver's; every other call accepts it too) on which
 * sinkhorn_init_norms has run.  Each call makes one pass over the keys with
 * lazily raised row offsets and recovers each row's log-sum-exp (for r_i) from
 * the offsets and weight sums.
 * --------------------------------------------------------------------------- */

/* Workspace bytes for the transport calls (0 if p is invalid). */
size_t sinkhorn_transport_workspace_bytes(const sk_problem* p);

sk_status sinkhorn_barycentric_x(const sk_problem* p, const void* X, const void* Y, void* ws,
                                 size_t ws_bytes, const float* f, const float* g, float eps,
                                 float* bary, float* grad, void* stream);

sk_status sinkhorn_barycentric_y(const sk_problem* p, const void* X, const void* Y, void* ws,
                                 size_t ws_bytes, const float* f, const float* g, float eps,
                                 float* bary, float* grad, void* stream);

/* ---------------------------------------------------------------------------
 * Plan application: vector- and matrix-transport products (page "FlashSinkhorn: Trasporto Ottimo
 * Entropico Consapevole delle I/O su GPU", section "Metodologia", part "3. Differenziazione e
 * Ottimizzazione del Secondo Ordine"), streamed like the transport calls, the plan never formed:
 *   sinkhorn_apply_plan_x:  out[b][i][k] = sum_j P_ij V[b][j][k]   V [batch][m][c] -> out [batch][n][c]
 *   sinkhorn_apply_plan_y:  out[b][j][k] = sum_i P_ij U[b][i][k]   U [batch][n][c] -> out [batch][m][c]
 * fp32 DEVICE arrays; c >= 1 columns.  c = 1 multiplies each fp32 weight with the
 * fp32 vector element on the vector unit; c > 1 is processed in passes of 64
 * columns, each value carried as three exact bf16 parts into the matrix product.
 * Workspace: sinkhorn_transport_workspace_bytes.
 * --------------------------------------------------------------------------- */
sk_status sinkhorn_apply_plan_x(const sk_problem* p, const void* X, const void* Y, void* ws,
                                size_t ws_bytes, const float* f, const float* g, float eps,
                                const float* V, int64_t c, float* out, void* stream);

sk_status sinkhorn_apply_plan_y(const sk_problem* p, const void* X, const void* Y, void* ws,
                                size_t ws_bytes, const float* f, const float* g, float eps,
                                const float* U, int64_t c, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * Hessian-vector products of the entropic OT value in the points (same page and
 * section: the HVP decomposes into transport products, with no Hessian and no
 * plan in memory; working memory O((n+m) d)).
 *   sinkhorn_hvp_x:  out = (d^2 OT / dX^2) V,  V and out [batch][n][d]
 *   sinkhorn_hvp_y:  out = (d^2 OT / dY^2) V,  V and out [batch][m][d]
 * at potentials (f, g) taken as optimal (pass the result of a converged solve).
 * Moving the points along V moves the potentials by (df, dg) that keep the plan's
 * marginals; df is eliminated and dg solves the Schur system
 * (diag(c) - P^T diag(1/r) P) dg = rhs by conjugate gradients (Jacobi
 * preconditioned, at most cg_iters iterations, stopped per problem when the
 * preconditioned residual falls below cg_tol relative to its start), each
 * iteration two one-column plan applications; the term sum_j P_ij (q_j . v_i) q_j
 * (q the other cloud) is one pass whose weights carry q_j . v_i.  Squared-Euclidean cost only
 * (SK_EUNSUPPORTED for the cosine cost).  Workspace: sinkhorn_hvp_workspace_bytes
 * (a superset of the transport workspace), after sinkhorn_init_norms.
 * --------------------------------------------------------------------------- */
size_t sinkhorn_hvp_workspace_bytes(const sk_problem* p);

sk_status sinkhorn_hvp_x(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                         const float* f, const float* g, float eps, const float* V, int64_t cg_iters,
                         float cg_tol, float* out, void* stream);

sk_status sinkhorn_hvp_y(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                         const float* f, const float* g, float eps, const float* V, int64_t cg_iters,
                         float cg_tol, float* out, void* stream);

/* Text for the last error on the calling thread ("" if none). */
const char* sinkhorn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SINKHORN_MI355X_H */
