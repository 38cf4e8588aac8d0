// Launchers of the HIP kernels of the primal path (gemm.hip, solve.hip).  All enqueue on `st` and
// return the launch status; none allocates or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dyra {

typedef __bf16 bf16;

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
// ldt).  float32 also writes Qt[b] = Q_b^T ([kc][npad], token-contiguous, zero
// for tokens n..npad-1); bf16 leaves Qt untouched.  flags[b] = 1 if a pivot
// broke down (then Q_b = 0).  kc in {16, 32, 48, 64}.
template <typename E>
hipError_t launch_gram_q(E *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real, int kc,
                         float lambda, E *Qt, int *flags, hipStream_t st);

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

}  // namespace dyra
