/*
 * sinkhorn.h -- C ABI of the MI355X (gfx950) streaming Sinkhorn library.
 *
 * Entropic optimal transport between point clouds under squared-Euclidean
 * cost, computed with stabilised log-domain Sinkhorn iterations in which every
 * half-iteration is one streamed row- or column-wise log-sum-exp of a biased
 * dot-product score; the n x m cost matrix never exists in memory.
 *
 * Sources, cited by page and section:
 *   [FS] "FlashSinkhorn: IO-bewuste Entropische Optimale Transport op GPU"
 *        (gist.science technical summary): Probleemstelling (problem: EOT
 *        between point clouds, squared-Euclidean cost); Methodologie 1,
 *        Propositie 1 (the f-update as the LSE of (Q K^T + 1(g_hat + delta))/eps,
 *        Q = sqrt2 X, K = sqrt2 Y); Methodologie 2 (tiles streamed, online
 *        max / sum-exp on chip, one fused pass per update, row-stationary).
 *   [AP] "From Theory to Throughput: CUDA-Optimized APML for Large-Batch 3D
 *        Learning" (newx.sg): Abstract and Innovation (negligible assignments
 *        thresholded away, plan kept in COO form, gradients on the stored
 *        support).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless the argument says "host".  Arrays
 *     are dense, row-major and batch-major: X[B][n][d], Y[B][m][d],
 *     a[B][n], b[B][m], f[B][n], g[B][m].  B pairs are independent problems
 *     of equal sizes.
 *   - X and Y share one dtype (SK_F32 or SK_BF16); everything else is fp32
 *     (indices int32, offsets int64).
 *   - The caller owns every buffer, including the workspace, whose size comes
 *     from sinkhorn_workspace_bytes().  The library allocates no device or
 *     pinned memory and keeps no state between calls, apart from a
 *     thread-local error message.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns without waiting, except sinkhorn_plan_coo and
 *     sinkhorn_coo_normalize, which read counts back (see there;
 *     sinkhorn_plan_coo_async is the plan without the wait).
 *     Calls are reentrant; two calls that share a workspace must not overlap.
 *   - Arguments are checked before anything is launched.  On an error no
 *     output buffer is written and the return value says why; the message
 *     of sinkhorn_last_error() gives detail.
 *   - Inputs are not scanned for NaN/Inf: NaN in gives NaN out.
 *   - Weights must be >= 0.  A zero weight removes that point from the other
 *     side's log-sum-exp (log 0 = -inf); its own potential stays defined.
 *     Each cloud of a pair needs at least one positive weight (the weights
 *     are not scanned: a cloud of zero mass gives meaningless potentials).
 *     a and b may be NULL, meaning uniform weights 1/n and 1/m.
 */
#ifndef SINKHORN_H
#define SINKHORN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
    SK_OK = 0,
    SK_ERR_INVALID_ARG = 1, /* a size, pointer, eps, threshold or flag is out of range */
    SK_ERR_UNSUPPORTED = 2, /* no kernel for this dtype / dimension combination */
    SK_ERR_WORKSPACE = 3,   /* ws is NULL or ws_bytes is below the required size */
    SK_ERR_CAPACITY = 4,    /* sparse plan larger than the caller's capacity */
    SK_ERR_HIP = 5          /* the HIP runtime reported an error (message has it) */
};

/* Point dtypes. */
enum { SK_F32 = 0, SK_BF16 = 1 };

/* Operation ids for sinkhorn_workspace_bytes(). */
enum {
    SK_OP_POTENTIALS = 0,
    SK_OP_PLAN_COO = 1,
    SK_OP_LOSS_GRAD = 2,
    SK_OP_DENSE_GRAD = 3,
    SK_OP_HVP = 4
};

/* Flags of sinkhorn_potentials(). */
#define SK_WARM_START 1u  /* f and g hold starting potentials (resume) */
#define SK_VALU_SCORES 2u /* d = 3: form scores on the vector ALUs instead of the
                             matrix cores (same results to fp32 rounding; slower
                             on gfx950, kept for comparison) */

/*
 * Supported shapes: 1 <= B <= 65535, 1 <= n, m <= 2^24, B*n and B*m <= 2^31, and
 *   d == 3, dtype SK_F32 or SK_BF16       (3-D point-cloud kernel), or
 *   dtype SK_F32 or SK_BF16, 1 <= d <= 128 (feature kernel; d is padded with
 *                                          zeros to the next of 8,16,32,64,128).
 * Anything else returns SK_ERR_UNSUPPORTED.
 */

/*
 * Bytes of workspace that operation `op` needs for these sizes (0 if the
 * arguments are out of range).  The value is an upper bound that depends only
 * on the arguments; the workspace needs no initialisation and its contents
 * are undefined after a call.
 */
size_t sinkhorn_workspace_bytes(int op, int B, int n, int m, int d, int dtype);

/*
 * Sinkhorn potentials [FS Methodologie 1, Propositie 1; Methodologie 2].
 *
 * For each stage s < n_stages (eps[s] > 0, iters[s] >= 0; both HOST arrays),
 * runs iters[s] full iterations, each an f-update followed by a g-update that
 * uses the new f:
 *     f_i <- -eps_s * LSE_j[(g_j - C_ij)/eps_s + log b_j]
 *     g_j <- -eps_s * LSE_i[(f_i - C_ij)/eps_s + log a_i],   C_ij = ||x_i - y_j||^2.
 * Potentials carry over from stage to stage (eps annealing).  Without
 * SK_WARM_START, g starts at 0 and f is not read; with it, f and g are read
 * as the starting point (resuming a split run gives the same result as one
 * long run).
 *
 * f [B][n], g [B][m] (fp32, in/out) receive the potentials after the last
 * g-update.  cost [B] (fp32, may be NULL) receives the transport cost
 * sum_ij P_ij C_ij of the plan at the last eps,
 *     log P_ij = (f_i + g_j - C_ij)/eps + log a_i + log b_j.
 * With n_stages == 0 (or all iters 0) the potentials are returned unchanged
 * (zero without SK_WARM_START) and cost is that of those potentials, at
 * eps[n_stages-1] if n_stages > 0; cost must be NULL when n_stages == 0.
 *
 * For d == 3, a small batch of clouds of at most 1024 points runs each stage
 * in one launch whose work-groups (at most half of the device's compute units)
 * wait for one another's results between half-iterations [FS Methodologie 2:
 * the update fused into as few launches as possible].  Those waits are
 * bounded: if the work-groups could not all run at once (the compute units
 * held by other work for about a second), the affected pairs' f and g come
 * back NaN instead of the call blocking.
 */
int sinkhorn_potentials(const void *X, const void *Y, int dtype,
                        const float *a, const float *b,
                        int B, int n, int m, int d,
                        const float *eps, const int *iters, int n_stages,
                        unsigned flags, float *f, float *g, float *cost,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * The same potentials with no workspace argument and no allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The caller passes inputs
 * and outputs as for sinkhorn_potentials; the workspace is a device array of
 * SK_NOALLOC_SCRATCH_BYTES bytes inside the library's code object, one copy per
 * GPU, held until the process ends.  Its address is resolved once per device,
 * on that device's first call (the current device; `stream` must belong to
 * it), so make the first call of each device outside any graph capture.
 *
 * Sizes whose workspace (sinkhorn_workspace_bytes(SK_OP_POTENTIALS, ...)) is
 * above SK_NOALLOC_SCRATCH_BYTES return SK_ERR_WORKSPACE with nothing written
 * (one pair of 65536 x 65536 points at d = 3 needs about 23 MiB; 256 pairs of
 * 1024 x 1024, 92 MiB).  The call allocates nothing (no hipMalloc or
 * allocating library routine) and launches the kernels of sinkhorn_potentials,
 * with the same results.  All calls on one GPU share its array: two calls that
 * overlap on one GPU (other streams, other threads) race and give undefined
 * results, so the caller must serialise them.  The array's contents need no
 * initialisation and are undefined after a call.
 */
#define SK_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int sinkhorn_potentials_noalloc(const void *X, const void *Y, int dtype,
                                const float *a, const float *b,
                                int B, int n, int m, int d,
                                const float *eps, const int *iters, int n_stages,
                                unsigned flags, float *f, float *g, float *cost,
                                void *stream);

/*
 * Thresholded sparse plan in COO form [AP Abstract, Innovation].
 *
 * From potentials f, g at eps (as returned by sinkhorn_potentials), keeps per
 * pair p every entry with
 *     P_ij >= rel_threshold * max_kl P_kl      (max over pair p; 0 < rel_threshold <= 1),
 * decided in the log domain.  Entries are written in (pair, row, column)
 * order without duplicates: rows[k], cols[k] (int32, indices within the
 * pair) and vals[k] = P_ij (fp32), for pair_offsets[p] <= k < pair_offsets[p+1].
 * pair_offsets has B+1 int64 entries (device).
 *
 * *nnz_total (HOST int64) always receives the number of kept entries.  If it
 * exceeds `capacity`, the call returns SK_ERR_CAPACITY after writing
 * pair_offsets and *nnz_total only; rows/cols/vals may be NULL when capacity
 * is 0.  The call synchronises `stream` once, to read the count back.
 *
 * loss [B] and dX [B][n][d] (fp32, device, each may be NULL) receive, in the
 * same pass, the transport loss on the emitted support and its gradient in X
 * with the plan held fixed [AP Abstract: gradients preserved on the stored
 * support]:
 *     loss[p] = sum_k vals_k ||x_{rows_k} - y_{cols_k}||^2,
 *     dX[p][i] = sum_{k: rows_k = i} 2 vals_k (x_i - y_{cols_k}),
 * i.e. what sinkhorn_loss_grad computes from the emitted plan, with the same
 * per-entry arithmetic (the summation order differs, so the two agree to
 * rounding).  Rows with no entry get a zero gradient.
 */
int sinkhorn_plan_coo(const void *X, const void *Y, int dtype,
                      const float *a, const float *b,
                      int B, int n, int m, int d, float eps,
                      const float *f, const float *g, float rel_threshold,
                      int64_t capacity, int32_t *rows, int32_t *cols, float *vals,
                      int64_t *pair_offsets, float *loss, float *dX, int64_t *nnz_total,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * The same plan (and optional loss / dX) without waiting on `stream`, for
 * callers that keep the host out of the loop (graph capture, training loops).
 * capacity >= 1 with rows/cols/vals of that many entries.  *nnz_device (DEVICE
 * int64) receives the number of kept entries and pair_offsets is written as
 * above.  If the count exceeds capacity nothing else is written: rows, cols,
 * vals, loss and dX keep their contents, so the caller must check
 * *nnz_device <= capacity before reading them (and call again with more room).
 * Launches kernels only (no copy, wait or memset).
 */
int sinkhorn_plan_coo_async(const void *X, const void *Y, int dtype,
                            const float *a, const float *b,
                            int B, int n, int m, int d, float eps,
                            const float *f, const float *g, float rel_threshold,
                            int64_t capacity, int32_t *rows, int32_t *cols, float *vals,
                            int64_t *pair_offsets, float *loss, float *dX, int64_t *nnz_device,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Loss and gradient on the stored support [AP Abstract] (plan held fixed):
 *     loss[p]  = sum_{k in pair p} vals_k * ||x_{rows_k} - y_{cols_k}||^2
 *     dX[p][i] = sum_{k in pair p, rows_k = i} 2 vals_k (x_i - y_{cols_k})
 * The COO must be in the form sinkhorn_plan_coo writes: within each pair,
 * entries sorted by row (any column order within a row), indices in range.
 * loss [B] fp32; dX [B][n][d] fp32 or NULL.  Rows with no entries get a
 * zero gradient.
 */
int sinkhorn_loss_grad(const void *X, const void *Y, int dtype,
                       int B, int n, int m, int d,
                       const int32_t *rows, const int32_t *cols, const float *vals,
                       const int64_t *pair_offsets, float *loss, float *dX,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Dense transport application: gradient and barycentric projection
 * [FS Methodologie 3, "Toepassing van Transportmatrix": both are weighted
 * averages over the plan, computed by streaming like the update, without
 * storing the plan].
 *
 * With the plan of potentials f, g at eps (the P of sinkhorn_potentials'
 * cost), for every point x_i of X and y_j of Y of each pair:
 *     dX[p][i] = sum_j 2 P_ij (x_i - y_j)          (gradient of sum P C in x_i,
 *     dY[p][j] = sum_i 2 P_ij (y_j - x_i)           P held fixed)
 *     TX[p][i] = sum_j P_ij y_j / sum_j P_ij       (barycentric projection)
 *     TY[p][j] = sum_i P_ij x_i / sum_i P_ij
 * dX, TX are [B][n][d] and dY, TY [B][m][d], fp32; each may be NULL, and a side
 * whose two outputs are both NULL is skipped.  A point whose row (column) of P
 * has zero mass gets a zero gradient and a zero projection.  log P is
 * evaluated in fp64 from the fp32 inputs, as for the sparse plan.
 */
int sinkhorn_dense_grad(const void *X, const void *Y, int dtype,
                        const float *a, const float *b,
                        int B, int n, int m, int d, float eps,
                        const float *f, const float *g,
                        float *dX, float *TX, float *dY, float *TY,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * Hessian-vector product of the entropic OT value in X [FS Methodologie 3,
 * Hessiaan-Vector Producten: transport-vector and transport-matrix products,
 * O((n+m)d) memory].
 *
 * HV = d/dt grad_X OT(X + t V) at t = 0, grad_i = sum_j 2 P_ij (x_i - y_j),
 * with P the plan of potentials f, g at eps (meant to be converged: the
 * derivative keeps P's row and column sums fixed, as they are at the solution).
 * The potentials' derivative solves a symmetric positive semidefinite m x m
 * system, (diag(mb) - P^T diag(1/ma) P) dg = c - P^T (r/ma), by `cg_iters`
 * conjugate-gradient steps from 0 (ma, mb: the plan's row and column sums;
 * r_i, c_j: row and column sums of P_ij 2 (x_i - y_j).v_i); every product with
 * P streams the plan, nothing n x m is stored.
 * V, HV: [B][n][d] fp32.  cg_residual [B] (device, may be NULL) receives the
 * final conjugate-gradient residual relative to the right-hand side.
 * Supported for d <= 16 (log P in fp64, either dtype) and for bf16 points with
 * d = 32 or 64 (SK_ERR_UNSUPPORTED otherwise).  The bf16 d = 32/64 path runs
 * every plan product on the matrix cores: plan entries from fp32 scores as in
 * the dense gradient, the direction V in two bf16 pieces (16 bits), fp32 sums;
 * it needs X and Y at 16-byte aligned addresses (SK_ERR_INVALID_ARG) and
 * potentials near the solution: a pair with a positive-weight row whose plan
 * mass, divided by its weight, falls outside [2^-64, 2^100] gets NaN in HV and
 * cg_residual.  Workspace sinkhorn_workspace_bytes(SK_OP_HVP, ...).
 */
int sinkhorn_hvp(const void *X, const void *Y, int dtype,
                 const float *a, const float *b,
                 int B, int n, int m, int d, float eps,
                 const float *f, const float *g, const float *V,
                 int cg_iters, float *HV, float *cg_residual,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * Sinkhorn normalisation of a sparse plan on its stored support [AP Abstract,
 * Innovation: Sinkhorn normalisation run directly in COO form].
 *
 * rows/cols/vals/pair_offsets: a plan as sinkhorn_plan_coo writes it (per pair
 * sorted by row, then column; B+1 offsets); t_rows/t_cols/t_vals/
 * t_pair_offsets: its transpose, i.e. the plan extracted with the roles of the
 * clouds exchanged (sinkhorn_plan_coo(Y, X, b, a, g, f, ...)), which holds
 * exactly the same entries and values because log P is evaluated
 * symmetrically.  Per pair, with lv = log vals, row scalings alpha and column
 * scalings beta start at 0 and each of `iters` rounds sets
 *     alpha_i = log a_i - LSE_{k in row i}(lv_k + beta_{col k}),
 *     beta_j  = log b_j - LSE_{k in col j}(lv_k + alpha_{row k})
 * (0 for a row or column without a finite term); then
 * vals_k <- exp(lv_k + alpha_{row k} + beta_{col k}) in place, in both the plan
 * and the transpose (which stay each other's transpose bit for bit): column
 * sums equal b, row sums approach a.  err [2B] (device, may be NULL) receives
 * per pair sum_i |row sum - a_i| and sum_j |column sum - b_j| of the result.
 * a, b may be NULL (uniform).  Workspace: sinkhorn_coo_workspace_bytes(B, n, m,
 * nnz).  Synchronises twice on `stream` (entry counts, transpose check).  The
 * transpose is checked per pair by entry count and by a 64-bit checksum of
 * every entry's (row, column, value bits); a mismatch returns
 * SK_ERR_INVALID_ARG with both value arrays unchanged.
 */
size_t sinkhorn_coo_workspace_bytes(int B, int n, int m, int64_t nnz);
int sinkhorn_coo_normalize(int B, int n, int m,
                           const int32_t *rows, const int32_t *cols, float *vals,
                           const int64_t *pair_offsets,
                           const int32_t *t_rows, const int32_t *t_cols, float *t_vals,
                           const int64_t *t_pair_offsets,
                           const float *a, const float *b, int iters, float *err,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Cosine cost on normalised vectors [FS Betekenis en Claims: the approach
 * applies to the cosine distance after normalisation].  For unit vectors
 * ||x^ - y^||^2 = 2 - 2 x^ . y^, so every entry point above, given the
 * normalised points, computes under the cosine cost; a gradient they return
 * (dX of sinkhorn_loss_grad or sinkhorn_dense_grad) is with respect to the
 * normalised points and sinkhorn_normalize_backward carries it to the raw ones.
 *
 * sinkhorn_normalize: Xh[B][n][d] = x / ||x|| (fp32), norms[B][n] = ||x||
 * (fp32), from X in `dtype` (SK_F32 or SK_BF16, any 1 <= d <= 4096); a zero
 * vector gives Xh = 0 and norm 0.  Norm and quotient in fp64, rounded once.
 * sinkhorn_normalize_backward: dX = (G - x^ (x^ . G)) / ||x|| for every point,
 * from Xh and norms as written above and G[B][n][d] (fp32); 0 for a zero
 * vector.  Both only enqueue work; no workspace.
 */
int sinkhorn_normalize(const void *X, int dtype, int B, int n, int d,
                       float *Xh, float *norms, void *stream);
int sinkhorn_normalize_backward(const float *Xh, const float *norms, const float *G,
                                int B, int n, int d, float *dX, void *stream);

/* Static text for a return code. */
const char *sinkhorn_status_string(int status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char *sinkhorn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SINKHORN_H */
