// BLAST static product, middle step (Appendix B of "DyRA: Dynamic Residual
// Approximation for Efficient Matrix Multiplication in DNNs").
//
// With W_hat's block (i, j) = U_i diag(s_ij) V_j^T, the static output of block
// column j is sum_i X_i U_i diag(s_ij) V_j^T.  The forward computes it in
// three steps: Z_i = X_i U_i (one GEMM per block row), H_j = sum_i Z_i
// diag(s_ij) (this kernel), Y_j = H_j V_j^T (one GEMM per block column, with
// the correction slices).  This kernel is elementwise across the rank index:
// for each token row and rank column c the nb values Z_i[c] are mixed by the
// nb x nb matrix s_..[c] into the nb values H_j[c], so it runs in place over
// T's first nb * rbp columns, and each thread owns its positions alone.
#include <hip/hip_runtime.h>

#include "dyra_kernels.h"
#include "mfma_tile.h"

namespace dyra {
namespace {

constexpr int kMixThreads = 256;

// Each thread holds one 16-byte chunk (VEC rank columns) of every block for
// one row, and keeps that chunk's couplings in registers while it walks rows.
template <typename E, int NB>
__global__ __launch_bounds__(kMixThreads) void blast_mix_kernel(E *__restrict__ T, int64_t ldt, int64_t N,
                                                                int rbp, const float *__restrict__ Smix) {
    constexpr int VEC = 16 / (int)sizeof(E);
    const int cpr = rbp / VEC;                // chunks per row and block
    const int rows_per_iter = kMixThreads / cpr;
    const int t = (int)threadIdx.x;
    if (t >= rows_per_iter * cpr) return;
    const int chunk = t % cpr, c0 = chunk * VEC;
    float s[NB][NB][VEC];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int v = 0; v < VEC; ++v) s[i][j][v] = Smix[((int64_t)i * NB + j) * rbp + c0 + v];
    const int64_t step = (int64_t)gridDim.x * rows_per_iter;
    for (int64_t row = (int64_t)blockIdx.x * rows_per_iter + t / cpr; row < N; row += step) {
        E *base = T + row * ldt + c0;
        u32x4 raw[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) raw[i] = *reinterpret_cast<const u32x4 *>(base + (int64_t)i * rbp);
        float z[NB][VEC];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const E *e = reinterpret_cast<const E *>(&raw[i]);
#pragma unroll
            for (int v = 0; v < VEC; ++v) z[i][v] = to_f32(e[v]);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            u32x4 out;
            E *o = reinterpret_cast<E *>(&out);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                float h = 0.f;
#pragma unroll
                for (int i = 0; i < NB; ++i) h = fmaf(z[i][v], s[i][j][v], h);
                o[v] = to_elem<E>(h);
            }
            *reinterpret_cast<u32x4 *>(base + (int64_t)j * rbp) = out;
        }
    }
}

template <typename E, int NB>
hipError_t mix_launch(E *T, int64_t ldt, int64_t N, int rbp, const float *Smix, hipStream_t st) {
    constexpr int VEC = 16 / (int)sizeof(E);
    const int rows_per_iter = kMixThreads / (rbp / VEC);
    const int64_t want = (N + rows_per_iter - 1) / rows_per_iter;
    const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
    hipLaunchKernelGGL((blast_mix_kernel<E, NB>), dim3(grid), dim3(kMixThreads), 0, st, T, ldt, N, rbp, Smix);
    return hipGetLastError();
}

}  // namespace

template <typename E>
hipError_t launch_blast_mix(E *T, int64_t ldt, int64_t N, int nb, int rbp, const float *Smix, hipStream_t st) {
    constexpr int VEC = 16 / (int)sizeof(E);
    if (N <= 0) return hipSuccess;
    if (rbp <= 0 || rbp % 32 != 0 || rbp / VEC > kMixThreads || ldt < (int64_t)nb * rbp || ldt % VEC != 0)
        return hipErrorInvalidValue;
    switch (nb) {
    case 1: return mix_launch<E, 1>(T, ldt, N, rbp, Smix, st);
    case 2: return mix_launch<E, 2>(T, ldt, N, rbp, Smix, st);
    case 3: return mix_launch<E, 3>(T, ldt, N, rbp, Smix, st);
    case 4: return mix_launch<E, 4>(T, ldt, N, rbp, Smix, st);
    }
    return hipErrorInvalidValue;
}

template hipError_t launch_blast_mix<bf16>(bf16 *, int64_t, int64_t, int, int, const float *, hipStream_t);
template hipError_t launch_blast_mix<float>(float *, int64_t, int64_t, int, int, const float *, hipStream_t);

}  // namespace dyra
