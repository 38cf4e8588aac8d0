// Launchers of the HIP kernels of the primal path (gemm.hip, solve.hip).  All enqueue on `st` and
// return the launch status; none allocates or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dyra {

typedef __bf16 bf16;

// One-time host set-up (dynamic LDS limits, resident workgroups per CU) of
// every GEMM instantiation on the current device, so that later launches only
// enqueue.  Launches that find their instantiation not set up do it first.
template <typename E> hipError_t gemm_prepare();
// The same for the BLAST mix kernels.
template <typename E> hipError_t blast_prepare();

// D[M][N] (leading dim ldd) = A[M][K] B[N][K]^T, K a multiple of 32.
template <typename E>
hipError_t launch_gemm_store(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                             E *D, int64_t ldd, hipStream_t st);

// R1t[b][c][kk] = alpha (Mp W_res)[b*kc + kk][c] for the stacked Mp [rows][c1].
template <typename E>
hipError_t launch_right(const E *Mp, const E *Wres_t, int64_t rows, int64_t c1, int64_t c2, int kc, float alpha,
                        E *R1t, hipStream_t st);

// With C C^T = L1_b^T L1_b + lambda I: Q_b = L1_b C^-T replaces L1_b in place
// (columns [off, off + kc) of T's rows b*n .. b*n + n - 1, leading dimension
// ldt).  float32 (kc <= 64) also writes Qt[b] = Q_b^T ([kc][npad],
// token-contiguous, zero for tokens n..npad-1); bf16 (kc <= 256) leaves Qt
// untouched and keeps C_b, column by column, in Ct ([B][kc][kc] float32
// workspace) between its two kernels, and, for kc above 128, G_b in Gw
// ([B] x gram_workspace_floats(kc) float32 workspace).  flags[b] = 1 if a
// pivot broke down (then Q_b = 0).  kc a multiple of 16.  Cout, if not null,
// receives the Cholesky factor C_b ([B][kc][kc] float64, lower, identity on
// the padding) for the L updates of further ALS steps.
template <typename E>
hipError_t launch_gram_q(E *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real, int kc,
                         float lambda, E *Qt, float *Ct, float *Gw, int *flags, double *Cout, hipStream_t st);
// Floats of the per-instance Gram buffer launch_gram_q<bf16> needs (0 if G
// stays in LDS).
size_t gram_workspace_floats(int kc);
// G_b = L1_b^T L1_b + lambda I alone (identity on the padding past kc_real),
// written whole to G ([B][kp][kp] float32, kp = kc rounded up to 32), for
// kc in 80..256 (the Newton-Schulz solve of large correction ranks).
template <typename E>
hipError_t launch_gram_only(const E *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int kc_real, int kc,
                            float lambda, float *G, hipStream_t st);

// Mp[b*kc + i][:] = (Q_b^T X_b)[i][:]: bf16 reads Q_b from T (as left by
// launch_gram_q), float32 from Qt.
template <typename E>
hipError_t launch_mprime(const E *X, const E *T, int64_t ldt, int64_t off, const E *Qt, int64_t B, int64_t n,
                         int64_t npad, int64_t c1, int kc, E *Mp, hipStream_t st);

// Y[Ntok][c2] = T[:, 0:kw] V_s^T + bias + T[:, kw:kw+kc] R1_b for each
// token's instance b (n tokens per instance; R1t[b] is [c2][kc]); T has
// leading dimension ldt; bias [c2] or null.  kc = 0 gives the static product
// (plus bias) alone.
template <typename E>
hipError_t launch_output(const E *T, int64_t ldt, int kw, int kc, const E *Vs, const E *R1t, int64_t Ntok,
                         int64_t n, int64_t c2, const E *bias, E *Y, hipStream_t st);

// The general form of launch_output: Y (leading dimension ldy) = A[:, 0:K]
// B^T + bias + A[:, kcol:kcol+kc] R1_b, where R1t + b * rstride is instance
// b's [N][kc] block; A and B have leading dimensions lda, ldb.  With
// gcols > 0 the static A operand is grouped: output columns
// [g gcols, g gcols + gcols) read A's columns from g * gstride on (the
// correction columns stay at kcol).  Used for a BLAST W_hat's block columns.
template <typename E>
hipError_t launch_output_ex(const E *A, int64_t lda, int64_t K, const E *B, int64_t ldb, int kcol, int kc,
                            const E *R1t, int64_t rstride, int64_t Ntok, int64_t n, int64_t N, const E *bias, E *Y,
                            int64_t ldy, int gcols, int64_t gstride, hipStream_t st);

// launch_gemm_store with a grouped A operand: D[:, g gcols .. g gcols +
// gcols - 1] = A[:, g gstride .. g gstride + K - 1] B[g gcols ..]^T.  One
// launch for a block-diagonal product.
template <typename E>
hipError_t launch_gemm_store_grouped(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N,
                                     int64_t K, int gcols, int64_t gstride, E *D, int64_t ldd, hipStream_t st);

// Whether an M x N product can be grouped in column groups of gcols (a tile
// shape that divides gcols exists).
bool gemm_groupable(int64_t M, int64_t N, int gcols);

// BLAST middle step (blast.hip): H_j = sum_i Z_i diag(s_ij) in place over
// T's columns [0, nb * rbp) (block i's Z, then block j's H, at columns
// [i rbp, i rbp + rbp)); Smix float32 [nb][nb][rbp].  nb <= 4, rbp a
// multiple of 32 with at most 256 16-byte chunks.
template <typename E>
hipError_t launch_blast_mix(E *T, int64_t ldt, int64_t N, int nb, int rbp, const float *Smix, hipStream_t st);

// Called after each kernel that a multi-kernel launcher enqueues: takes the
// launch status, records the next timing event (if any) on the stream, and
// returns the status to go on with.
struct EventMark {
    void *const *events = nullptr;
    int32_t n_events = 0;
    int32_t *count = nullptr;
    hipStream_t st = nullptr;
    hipError_t operator()(hipError_t e) const {
        if (e != hipSuccess) return e;
        if (events && count && *count < n_events) {
            e = hipEventRecord((hipEvent_t)events[*count], st);
            ++*count;
        }
        return e;
    }
};

// Column ranges over which the Gram matrix R' R'^T of an L update is split.
constexpr int kAlsGramSplit = 8;

// Buffers of one L update of a further ALS step (als.hip).  kc is the padded
// correction rank (16..64), k_real the requested one.
template <typename E> struct AlsArgs {
    const E *X;          // [B*n][c1]
    int64_t B, n, c1, c2;
    int kc, k_real;
    float lambda;
    const E *R1t;        // [B][c2][kc]  R' of the previous R update (unscaled)
    E *R1row;            // [B*kc][c2]   R' by rows (workspace)
    const E *Wres;       // [c1][c2]     W_res, row-major
    E *Sp;               // [B*kc][c1]   S'^T = R' W_res^T (workspace)
    float *H;            // [kAlsGramSplit][B][kc][kc]  partial sums of R' R'^T (workspace)
    const double *C;     // [B][kc][kc]  Cholesky factor of the previous R update
    float *Kp;           // [B][kc][kc]  K' (workspace)
    int *flags;          // [B]          set to 1 where the L update broke down
    E *T;                // left-pass buffer; the new L goes to columns [off, off + kc)
    int64_t ldt, off;
};

// One L update (Eq. 4) for every instance, as five kernels (transpose of R',
// S' GEMM, H', K', L), each followed by mark().  last = 1: the update is the
// final one, and the L columns receive alpha X S' Z^-1 (to be multiplied by
// R' in the output); last = 0: they receive the new L = X S' Z^-1 C^T.
template <typename E>
hipError_t launch_als_lupdate(const AlsArgs<E> &a, int last, float alpha, hipStream_t st, const EventMark &mark);

// §2.4's Newton-Schulz alternative to launch_gram_q (ns.hip): G = L1^T L1 +
// lambda I per instance, F = G^-1/2 by `iters` coupled Newton-Schulz steps
// (F [B][kc][kc] float32, workspace), then Q = L1 F in place in T's columns
// [off, off + kc) (float32 plans also fill Qt as launch_gram_q does).
// flags[b] = 1 where F is not finite (the correction is then dropped).  Two
// kernels, each followed by mark().
// Floats of the Newton-Schulz workspace F of launch_ns_solve: F_b [kc][kc]
// per instance for kc <= 64; the iterates Y, Z (two each), T ([kp][kp] per
// instance) and the scale c per instance above.
size_t ns_workspace_floats(int64_t B, int kc);
template <typename E>
hipError_t launch_ns_solve(E *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real, int kc,
                           float lambda, int iters, float *F, int *flags, float *Qt, hipStream_t st,
                           const EventMark &mark);

}  // namespace dyra
