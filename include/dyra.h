/*
 * libdyra -- DyRA's one-step dynamic residual approximation of a linear layer
 * on AMD Instinct MI355X (gfx950).
 *
 * Method: "DyRA: Dynamic Residual Approximation for Efficient Matrix
 * Multiplication in DNNs" (Chae, Chung, Lee, Kim).  For a layer Y = X W with
 * W in R^{c1 x c2}, the library computes
 *
 *     Y_hat = (X A_s) V_s^T + L1 R1                       (§2.3 Eq. 6, Prop. 1 Eq. 8)
 *
 * where W_hat = A_s V_s^T is the rank-r truncated SVD of W (Appendix B, with
 * the singular values folded into A_s), W_res = W - W_hat (§2.1 Eq. 1), and per
 * instance (a block of n consecutive token rows, §2.4) the correction factors
 * are one ALS step on min ||X W_res - L R||_F (§2.2 Eq. 3-5, Algorithm 1):
 *
 *     L1 = X P_L,  P_L = W_res R0^T (R0 R0^T + lambda I)^-1   (Eq. 7)
 *     R1 = (L1^T L1 + lambda I)^-1 (L1^T X) W_res              (Eq. 5)
 *
 * with R0 the top-k right singular vectors of W_res (Appendix D).  "r" is the
 * static (weight) rank and "k" the correction rank throughout this header.
 *
 * All entry points are C99, take plain pointers and sizes, and return a
 * dyra_status.  None throws, aborts or prints.  Argument checks run on the host
 * before anything is enqueued, so they can be exercised without a GPU.
 */
#ifndef DYRA_H
#define DYRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DYRA_OK = 0,
    DYRA_ERR_ARG = 1,        /* null pointer, bad rank, negative or non-finite lambda */
    DYRA_ERR_SHAPE = 2,      /* a dimension the kernels do not support (see each call) */
    DYRA_ERR_DTYPE = 3,      /* unknown dtype */
    DYRA_ERR_ALIGN = 4,      /* a device pointer not 16-byte aligned */
    DYRA_ERR_NUMERIC = 5,    /* non-finite weight, or a factorisation that did not converge */
    DYRA_ERR_HIP = 6,        /* a HIP runtime call or kernel launch failed */
    DYRA_ERR_NOMEM = 7,      /* host or device allocation failed */
    DYRA_ERR_WORKSPACE = 8,  /* workspace missing or smaller than dyra_workspace_bytes() */
    DYRA_ERR_NODEVICE = 9,   /* no HIP device, or the plan lives on another device */
    DYRA_ERR_SCRATCH = 10    /* dyra_forward_noalloc: the call needs more than its built-in scratch */
} dyra_status;

typedef enum {
    DYRA_F32 = 0,   /* float32 operands, float32 accumulation */
    DYRA_BF16 = 1   /* bfloat16 operands and stored intermediates, float32 accumulation */
} dyra_dtype;

/* Opaque prepared layer.  Owns its device buffers; immutable after dyra_prepare,
   so several streams may run dyra_forward on one plan at once, each with its own
   workspace. */
typedef struct dyra_plan dyra_plan;

/* Human-readable name of a status code (static storage, never NULL). */
const char *dyra_status_str(dyra_status s);

/*
 * Offline factorisation, host only (Algorithm 1, Offline Preparation, lines 2-5;
 * Appendix B truncated SVD; Appendix D choice of R0; Eq. 7).
 *
 * W       host, float32, row-major [c1][c2] in the X W orientation (an nn.Linear
 *         weight is [c2][c1]: pass its transpose).  Not modified, not retained.
 * r, k    static rank >= 0 and correction rank >= 0, r + k <= min(c1, c2).
 * lambda  ridge term >= 0 used in both Gram matrices (§2.2 footnote 2).
 * Outputs (host, float64, caller-owned; any may be NULL to skip it):
 *   A_s   [c1][r]   U_r diag(sigma_r), row-major
 *   V_s   [c2][r]   V_r, row-major
 *   R0    [k][c2]   V_{r+1..r+k}^T, row-major (orthonormal rows)
 *   P_L   [c1][k]   W_res R0^T (R0 R0^T + lambda I)^-1, row-major
 *   sigma [r + k]   leading singular values of W, descending
 * The SVD is formed from the float64 Gram matrix on the smaller side and a
 * symmetric eigensolver (Householder tridiagonalisation, bisection, inverse
 * iteration).  Returns DYRA_ERR_NUMERIC for a non-finite W.  No HIP call is made.
 */
dyra_status dyra_factorize_host(const float *W, int64_t c1, int64_t c2, int32_t r, int32_t k,
                                double lambda, double *A_s, double *V_s, double *R0,
                                double *P_L, double *sigma);

/*
 * Algorithm 1, Offline Preparation: factorise W on the host (as
 * dyra_factorize_host), round the factors to `dtype` (round to nearest even),
 * pack them in the kernels' layouts and copy them to `device`.  Synchronous;
 * not on the timed path.
 *
 * W, c1, c2, r, k, lambda as for dyra_factorize_host.  c1 and c2 must be
 * multiples of 32 (DYRA_ERR_SHAPE otherwise).  r and k may be any values with
 * r + k <= min(c1, c2) and k <= 256 (k <= 64 for DYRA_F32; DYRA_ERR_SHAPE
 * otherwise); k = 0 gives the weight-only product X A_s V_s^T, and
 * r = min(c1, c2), k = 0 the exact product up to rounding.
 * On success *plan_out owns device memory until dyra_plan_destroy: for k > 0,
 * W_res^T, V_s and [A_s | P_L] twice (row-major for the primal path, and in
 * MFMA fragment order for the dual form of short instances), about
 * 2 (c1 c2 + (r + k) c1 + c2 r) elements of `dtype`.
 */
dyra_status dyra_prepare(const float *W, int64_t c1, int64_t c2, int32_t r, int32_t k,
                         float lambda, dyra_dtype dtype, int device, dyra_plan **plan_out);

/*
 * dyra_prepare with the method's further knobs (§2.2 Fig. 2 / Appendix E.3
 * Gaussian R^(0); §3.3 ablation over the ALS iteration count t; §2.4
 * Newton-Schulz SPD solve):
 *
 * R0              host, float32, row-major [k][c2], caller-owned, not retained;
 *                 used as R^(0) in P_L = W_res R0^T (R0 R0^T + lambda I)^-1
 *                 (Eq. 7) in place of the top-k right singular vectors of W_res.
 *                 NULL keeps the default (Appendix D).  Non-finite entries give
 *                 DYRA_ERR_NUMERIC, a rank-deficient R0 with lambda = 0 as well.
 * als_half_steps  number of single ALS updates, alternating L (Eq. 4) and R
 *                 (Eq. 5) from R^(0): 2 = one iteration, t = 1 (Algorithm 1,
 *                 dyra_prepare's choice), 3 = t 1.5 (L, R, L), 4 = t 2, up to 8;
 *                 DYRA_ERR_ARG outside [2, 8].  The output is the product of the
 *                 last L and the last R.  Ignored when k = 0.
 * ns_iters        0: the SPD system of Eq. 5 is solved by Cholesky (§2.4's
 *                 choice for small r).  1..64: by that many steps of the
 *                 coupled Newton-Schulz iteration for G^-1/2 (§2.4's choice for
 *                 large r): c = ||G||_F, Y = G / c, Z = I, T = (3I - Z Y) / 2,
 *                 Y <- Y T, Z <- T Z, F = Z / sqrt(c), Q = L1 F.  Requires
 *                 als_half_steps = 2 (DYRA_ERR_ARG otherwise).  An instance
 *                 whose F is not finite is flagged (dyra_forward_status) and
 *                 gets no correction.  The dual form does not use it.
 *
 * A plan with als_half_steps > 2 also holds W_res untransposed ([c1][c2]) and
 * needs a larger workspace; dyra_forward runs the extra steps for instances
 * on the primal path (n > 16 tokens with n >= k, or n < k with lambda > 0) and
 * returns DYRA_ERR_SHAPE for the dual form, which carries one ALS step only.
 * als_half_steps > 2 takes k <= 64 (DYRA_ERR_SHAPE above).  With ns_iters > 0
 * and k above 64 the correction rank is padded to a multiple of 64 and each
 * Newton-Schulz product runs for all instances at once on float32 MFMA.
 */
dyra_status dyra_prepare_ex(const float *W, int64_t c1, int64_t c2, int32_t r, int32_t k, float lambda,
                            dyra_dtype dtype, int device, const float *R0, int32_t als_half_steps,
                            int32_t ns_iters, dyra_plan **plan_out);

/*
 * The host part of dyra_prepare_blast alone, for checking it without a GPU:
 * W_res = W - W_hat [c1][c2], R0 [k][c2] and P_L [c1][k] (float64, row-major,
 * caller-owned; any output may be NULL).  Arguments and errors as for
 * dyra_prepare_blast, without the device, dtype and shape-limit checks.
 */
dyra_status dyra_factorize_blast_host(const float *W, int64_t c1, int64_t c2, int32_t nb, int32_t rb,
                                      const float *U, const float *S, const float *V, int32_t k,
                                      double lambda, double *W_res, double *R0, double *P_L);

/*
 * Algorithm 1, Offline Preparation, with a BLAST structured approximation in
 * place of the truncated SVD (Appendix B, BLAST; §1 and §2.3 pair DyRA with
 * any structured W_hat).  W is cut into an nb x nb grid of (c1/nb) x (c2/nb)
 * blocks, and block (i, j) of W_hat is U_i diag(s_ij) V_j^T.  The block
 * coupling is taken as diagonal: the paper leaves its shape ambiguous, and
 * only the diagonal form reaches the FLOPs reductions it reports for the
 * BLAST ranks it sweeps.  The paper fits the factors by minimising
 * ||W - W_hat||_F and leaves the method open, so the caller supplies them.
 *
 * W   host float32 row-major [c1][c2] (X @ W orientation), as for dyra_prepare.
 * U   host float32 row-major [c1][rb]: rows i*c1/nb .. (i+1)*c1/nb - 1 are U_i.
 * S   host float32 [nb][nb][rb]: S[i][j][:] = s_ij, the diagonal of block (i, j).
 * V   host float32 row-major [c2][rb]: rows j*c2/nb .. (j+1)*c2/nb - 1 are V_j.
 * nb  1..4 blocks per side; c1 and c2 multiples of 32 * nb.
 * rb  BLAST rank >= 1; padded to 32 it must fit 256 16-byte chunks (rb <= 2048
 *     for bf16, 1024 for float32).
 * k   correction rank 0..256 (0..64 for DYRA_F32), k <= min(c1, c2); lambda >= 0
 *     and finite.
 *
 * W_res = W - W_hat, R0 = the top-k right singular vectors of W_res
 * (Appendix D) and P_L (Eq. 7) are formed on the host in float64.  The
 * forward runs the static product as X_i U_i per block row, the mix
 * H_j = sum_i (X_i U_i) diag(s_ij), and H_j V_j^T per block column, with the
 * correction added in the block-column products.  One ALS step with the
 * Cholesky solve; no dual form: with lambda = 0 a forward with fewer tokens per
 * instance than k returns DYRA_ERR_SHAPE.  dyra_plan_info reports r = rb.
 * Errors as dyra_prepare, plus DYRA_ERR_SHAPE for nb, rb or dimensions out of
 * range; DYRA_ERR_NUMERIC for non-finite factors.  The factors are read
 * during the call only.
 */
dyra_status dyra_prepare_blast(const float *W, int64_t c1, int64_t c2, int32_t nb, int32_t rb,
                               const float *U, const float *S, const float *V, int32_t k, float lambda,
                               dyra_dtype dtype, int device, dyra_plan **plan_out);

/* Releases a plan and its device memory.  NULL is ignored. */
void dyra_plan_destroy(dyra_plan *plan);

/* Dimensions of a plan (any output pointer may be NULL). */
dyra_status dyra_plan_info(const dyra_plan *plan, int64_t *c1, int64_t *c2, int32_t *r,
                           int32_t *k, float *lambda, dyra_dtype *dtype, int *device);

/*
 * Device workspace that dyra_forward needs for B instances of n tokens.
 * Returns 0 for a NULL plan, B < 0 or n < 1.  The workspace holds one int32
 * failure flag per instance, the left pass output [X A_s | L1] (L1 later
 * replaced by Q = L1 C^-T, C C^T = L1^T L1 + lambda I), M' = Q^T X and R1 per
 * instance (for float32 also Q^T), or the dual form's buffers when n <= 16 or
 * n < k.  For a BLAST plan the left pass output is [H_1 .. H_nb | L1], the
 * block-column inputs of the static product, and there is no dual form.
 */
size_t dyra_workspace_bytes(const dyra_plan *plan, int64_t B, int64_t n);

/*
 * Algorithm 1, Inference (lines 10-13), for B independent instances of n tokens.
 *
 * X          device, plan dtype, row-major [B*n][c1]; instance b is rows [b*n, b*n+n).
 * Y          device, plan dtype, row-major [B*n][c2]; fully overwritten.
 * workspace  device, >= dyra_workspace_bytes(plan, B, n) bytes, caller-owned,
 *            contents on entry ignored.  Calls that overlap in time need
 *            separate workspaces.
 * stream     a hipStream_t (NULL = the default stream) on the plan's device.
 * All pointers 16-byte aligned.  B >= 0, n >= 1 (B = 0 is a no-op).
 *
 * Asynchronous: enqueues kernels on `stream` and returns; no allocation, no
 * host synchronisation.  For n > 16 and n >= k (or n < k with lambda > 0) the
 * per-instance right factor comes from a Cholesky factorisation of
 * L1^T L1 + lambda I (§2.4); for n <= 16, and for 16 < n < k with lambda = 0,
 * the same product L1 R1 is formed in its n x n dual (push-through) form
 * L1 L1^T (L1 L1^T + lambda I_n)^-1 X W_res, which is also defined at
 * lambda = 0 (the projector onto the range of L1, by an eigen-decomposition
 * for n <= 16 and a Cholesky factorisation with diagonal pivoting for
 * 16 < n <= 64) and better conditioned when n is close to k.  lambda = 0 with
 * 64 < n < k returns DYRA_ERR_SHAPE.  A
 * Cholesky pivot at or below the working precision (lambda = 0 with a
 * numerically rank-deficient L1) sets that instance's failure flag, read back
 * by dyra_forward_status(); its rows then hold the static product X A_s V_s^T
 * alone.  Every call that forms a correction rewrites every flag; the
 * weight-only path (k = 0) writes none, and dyra_forward_status reports no
 * failure for it.  The kernels' one-time host set-up (LDS limits, resident
 * workgroups per CU) is done by the preparation calls on the plan's device,
 * so a forward call on a prepared device makes no HIP call besides its kernel
 * launches and can be captured into a graph.  A BLAST plan (dyra_prepare_blast)
 * always takes the k x k Cholesky form and returns DYRA_ERR_SHAPE for n < k
 * with lambda = 0; its static product is X W_hat for the BLAST W_hat.
 */
dyra_status dyra_forward(const void *X, int64_t B, int64_t n, const dyra_plan *plan, void *Y,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The fused linear layer of §2.4: as dyra_forward, but
 *     Y = X A_s V_s^T + bias + alpha L1 R1
 * per instance, with the bias added to every row and alpha weighting only the
 * dynamic correction (alpha = 1 and no bias is Eq. 6 / dyra_forward).
 *
 * bias   device, plan dtype, [c2], caller-owned, or NULL for none; aligned to
 *        its element size (DYRA_ERR_ALIGN otherwise).
 * alpha  finite (DYRA_ERR_ARG otherwise); 0 gives the static product plus bias.
 * Everything else, including the paths taken and the failure flags, as for
 * dyra_forward.  The bias is added in float32 before the single rounding of Y.
 */
dyra_status dyra_forward_ex(const void *X, int64_t B, int64_t n, const dyra_plan *plan, const void *bias,
                            float alpha, void *Y, void *workspace, size_t workspace_bytes, void *stream);

/*
 * dyra_forward for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and result as dyra_forward, with the
 * workspace taken from a scratch array built into the library, one per GPU,
 * of dyra_noalloc_scratch_bytes() (128 MiB) and held until the process ends.
 * No allocation or free of any kind is made.
 *
 * X, Y, plan, stream, B, n as for dyra_forward.  Returns DYRA_ERR_SCRATCH when
 * dyra_workspace_bytes(plan, B, n) exceeds the scratch (nothing is enqueued),
 * DYRA_ERR_NODEVICE if no plan was prepared on the plan's device in this
 * process.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  The scratch keeps the last call's contents; no
 * kernel reads it before writing it.  dyra_forward_status does not see this
 * call's failure flags.
 */
dyra_status dyra_forward_noalloc(const void *X, int64_t B, int64_t n, const dyra_plan *plan, void *Y,
                                 void *stream);

/* Size in bytes of dyra_forward_noalloc's per-GPU scratch. */
size_t dyra_noalloc_scratch_bytes(void);

/*
 * Number of instances whose SPD solve broke down in the last
 * dyra_forward(X, B, n, plan, ...) that used this workspace.  Copies the B
 * flags from the workspace on `stream` and synchronises it; *failures
 * receives the count.  For the weight-only path (k = 0) it is 0 without a
 * copy.
 */
dyra_status dyra_forward_status(const dyra_plan *plan, int64_t B, int64_t n, const void *workspace,
                                void *stream, int32_t *failures);

/*
 * The exact product Y = X W (§2.1 Eq. 2) for parity checks and as the dense
 * timing point.  X device [N][c1], Wt device [c2][c1] (W transposed, i.e. the
 * nn.Linear weight layout), Y device [N][c2], all in `dtype`, row-major,
 * 16-byte aligned; float32 accumulation.  c1 and c2 multiples of 32.
 * Asynchronous on `stream`.  The first call on a device where no plan was
 * prepared also does the GEMM kernels' one-time host set-up.
 */
dyra_status dyra_dense_ref(const void *X, const void *Wt, int64_t N, int64_t c1, int64_t c2,
                           dyra_dtype dtype, void *Y, void *stream);

/*
 * Stage timing for measurement tools: as dyra_forward, but records
 * events[0..n_events) (hipEvent_t, created by the caller) on `stream` before
 * the first kernel and after each kernel of the path.  *n_recorded receives the
 * number of events used (stages + 1, at most n_events).  Stage names are
 * returned by dyra_stage_name().
 */
dyra_status dyra_forward_timed(const void *X, int64_t B, int64_t n, const dyra_plan *plan,
                               void *Y, void *workspace, size_t workspace_bytes, void *stream,
                               void *const *events, int32_t n_events, int32_t *n_recorded);

/* Name of stage i of the path dyra_forward takes for (plan, n); NULL past the end. */
const char *dyra_stage_name(const dyra_plan *plan, int64_t n, int32_t i);

#ifdef __cplusplus
}
#endif

#endif /* DYRA_H */
