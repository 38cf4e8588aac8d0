// Further alternating-least-squares steps on the primal path (gfx950).
//
// "DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
// DNNs", Eq. 3-5 and the §3.3 ablation over the ALS iteration count t
// (t = 1.5 adds one L update after Algorithm 1's L, R; t = 2 adds an L and an
// R update).  The R update is the one Algorithm 1 line 12 already takes
// (launch_gram_q, launch_mprime, launch_right); this file holds the L update
// of Eq. 4,
//     L <- X W_res R^T (R R^T + lambda I)^-1,
// for every instance, in terms of what the R update leaves behind: the
// Cholesky factor C of L^T L + lambda I and R' = Q^T X W_res with
// Q = L C^-T, so that R = C^-T R'.  With S' = W_res R'^T (c1 x k) and
// H' = R' R'^T,
//     W_res R^T = S' C^-1,   R R^T = C^-T H' C^-1,
//     L_new = X S' Z^-1 C^T,  Z = H' + lambda C^T C,
// and the product the output needs when the L update is the last one is
//     L_new R = X S' Z^-1 R'.
// So one L update is: R' rows (a transpose of the stored R1t), the GEMM
// S'^T = R' W_res^T (launch_gemm_store), H' per instance, the k x k matrix
// K' = Z^-1 C^T (or Z^-1 for the last update) per instance in float64,
// P = K'^T-weighted rows of S', and L_new = X_b P_b^T into the L columns of
// the left-pass buffer.
#include "dyra_kernels.h"

#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;

// R1row[b][kk][c] = R1t[b][c][kk]; 64 columns c per workgroup through LDS.
template <typename E>
__global__ __launch_bounds__(NT) void transpose_r1_kernel(const E *__restrict__ R1t, int64_t c2, int kc,
                                                          E *__restrict__ R1row) {
    __shared__ E tile[64][64 + 1];  // [c][kk]
    const int64_t b = blockIdx.y, c0 = (int64_t)blockIdx.x * 64;
    const E *src = R1t + (b * c2 + c0) * kc;
    for (int e = threadIdx.x; e < 64 * kc; e += NT) {
        const int c = e / kc, kk = e - c * kc;
        if (c0 + c < c2) tile[c][kk] = src[(int64_t)c * kc + kk];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * kc; e += NT) {
        const int kk = e >> 6, c = e & 63;
        if (c0 + c < c2) R1row[(b * kc + kk) * c2 + c0 + c] = tile[c][kk];
    }
}

// H[b] = R'_b R'_b^T ([kc][kc] float32) from the kc rows of R1row that belong
// to instance b (length c2).  One workgroup per instance, one 32 x 32 block of
// H per wavefront; rows past kc read as zero.
template <typename E>
__global__ __launch_bounds__(NT) void gram_rows_kernel(const E *__restrict__ R1row, int64_t c2, int kc,
                                                       float *__restrict__ H) {
    typedef typename Frag<E>::type F;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t b = blockIdx.x;
    const int nb = (kc + 31) / 32;
    if (wm >= nb || wn >= nb) return;  // the kernel has no barrier
    const int ri = wm * 32 + lr, rj = wn * 32 + lr;
    const E *pa = R1row + (b * kc + (ri < kc ? ri : 0)) * c2;
    const E *pb = R1row + (b * kc + (rj < kc ? rj : 0)) * c2;
    f32x16 acc = f32x16{};
#pragma unroll 4
    for (int64_t c = 0; c < c2; c += 16) {
        const F fa = ri < kc ? ld_frag(pa + c + lk) : F{};
        const F fb = rj < kc ? ld_frag(pb + c + lk) : F{};
        acc = mma16(acc, fa, fb);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int row = wm * 32 + acc_row(lane, q), col = rj;
        if (row < kc && col < kc) H[(b * kc + row) * kc + col] = acc[q];
    }
}

// K'_b ([kc][kc] float32) from H'_b and C_b, in float64:
//   Z = H' + lambda C^T C on the real indices (identity on the padding),
//   Z = D D^T (Cholesky), Z^-1 = D^-T D^-1,
//   K' = Z^-1 C^T (the L update is followed by an R update: rows of P are
//   then the columns of L_new = X S' K'), or alpha Z^-1 (the last update:
//   L_new R = X S' Z^-1 R', alpha weighting the correction).
// A pivot of Z at or below kc times float32 precision times its largest
// diagonal entry (possible only for lambda = 0, when R' is rank deficient)
// sets flags[b] and makes K' zero: the instance then gets no correction.
__global__ __launch_bounds__(NT) void als_coef_kernel(const float *__restrict__ H, const double *__restrict__ C,
                                                      int kc, int kc_real, float lambda, int last, float alpha,
                                                      float *__restrict__ Kp, int *__restrict__ flags) {
    __shared__ double Z[64][65];
    __shared__ double Di[64][65];
    __shared__ double Cs[64][65];
    __shared__ int fail;
    __shared__ double thresh;
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    for (int e = tid; e < kc * kc; e += NT) {
        const int i = e / kc, j = e - i * kc;
        Cs[i][j] = C[b * kc * kc + e];
    }
    if (tid == 0) fail = 0;
    __syncthreads();
    for (int e = tid; e < kc * kc; e += NT) {
        const int i = e / kc, j = e - i * kc;
        double z;
        if (i < kc_real && j < kc_real) {
            double s = 0.0;
            for (int m = 0; m < kc; ++m) s += Cs[m][i] * Cs[m][j];
            z = (double)H[b * kc * kc + e] + (double)lambda * s;
        } else {
            z = i == j ? 1.0 : 0.0;
        }
        Z[i][j] = z;
    }
    __syncthreads();
    if (tid == 0) {
        double dmax = 0.0;
        for (int i = 0; i < kc_real; ++i) dmax = Z[i][i] > dmax ? Z[i][i] : dmax;
        thresh = lambda > 0.f ? 0.0 : (double)kc * 1.2e-7 * dmax;
        if (!(dmax > 0.0)) fail = 1;
    }
    __syncthreads();
    // ---- Z = D D^T, right-looking, lower triangle of Z
    for (int K = 0; K < kc; ++K) {
        if (tid == 0) {
            double pk = Z[K][K];
            if (K < kc_real && !(pk > thresh)) {
                fail = 1;
                pk = 1.0;
            }
            Z[K][K] = sqrt(pk);
        }
        __syncthreads();
        const double d = Z[K][K];
        for (int i = K + 1 + tid; i < kc; i += NT) Z[i][K] /= d;
        __syncthreads();
        const int w = kc - K - 1;
        for (int e = tid; e < w * w; e += NT) {
            const int i = K + 1 + e / w, j = K + 1 + e % w;
            if (j <= i) Z[i][j] -= Z[i][K] * Z[j][K];
        }
        __syncthreads();
    }
    // ---- D^-1 (lower), one column per thread by forward substitution
    if (tid < kc) {
        const int j = tid;
        for (int i = 0; i < kc; ++i) {
            double v;
            if (i < j) {
                v = 0.0;
            } else {
                double s = i == j ? 1.0 : 0.0;
                for (int m = j; m < i; ++m) s -= Z[i][m] * Di[m][j];
                v = s / Z[i][i];
            }
            Di[i][j] = v;
        }
    }
    __syncthreads();
    // ---- Z^-1 = D^-T D^-1 into Z (D is no longer needed)
    for (int e = tid; e < kc * kc; e += NT) {
        const int i = e / kc, j = e - i * kc;
        const int m0 = i > j ? i : j;
        double s = 0.0;
        for (int m = m0; m < kc; ++m) s += Di[m][i] * Di[m][j];
        Z[i][j] = s;  // D is not read here: only D^-1
    }
    __syncthreads();
    const bool failed = fail != 0;
    for (int e = tid; e < kc * kc; e += NT) {
        const int i = e / kc, j = e - i * kc;
        double v;
        if (last) {
            v = (double)alpha * Z[i][j];
        } else {
            // (Z^-1 C^T)[i][j] = sum_m Z^-1[i][m] C[j][m]
            double s = 0.0;
            for (int m = 0; m <= j; ++m) s += Z[i][m] * Cs[j][m];
            v = s;
        }
        Kp[b * kc * kc + e] = failed ? 0.f : (float)v;
    }
    if (tid == 0 && failed) flags[b] = 1;
}

// P[b*kc + kk][f] = sum_j K'_b[j][kk] S'[b*kc + j][f]: the coefficient rows
// of the new L (L_new = X_b P_b^T).  Workgroup (256 input features, instance
// b), one feature per thread, K'_b in LDS.
template <typename E, int KC>
__global__ __launch_bounds__(NT) void als_apply_kernel(const float *__restrict__ Kp, const E *__restrict__ Sp,
                                                       int64_t c1, E *__restrict__ P) {
    __shared__ float Ks[KC][KC];  // Ks[j][kk] = K'[j][kk]
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t f = (int64_t)blockIdx.x * NT + tid;
    for (int e = tid; e < KC * KC; e += NT) (&Ks[0][0])[e] = Kp[b * KC * KC + e];
    __syncthreads();
    if (f >= c1) return;
    float p[KC];
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) p[kk] = 0.f;
    const E *s0 = Sp + b * KC * c1 + f;
    for (int j = 0; j < KC; ++j) {
        const float s = (float)s0[(int64_t)j * c1];
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) p[kk] = fmaf(Ks[j][kk], s, p[kk]);
    }
    E *p0 = P + b * KC * c1 + f;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) p0[(int64_t)kk * c1] = to_elem<E>(p[kk]);
}

// T[b*n + t][off + kk] = sum_f X[b*n + t][f] P[b*kc + kk][f]: the new L of
// instance b in the L columns of the left-pass buffer.  Workgroup (64 tokens,
// instance b), one 32 x 32 block per wavefront, operands straight from global
// memory (16-byte fragments along f).
template <typename E>
__global__ __launch_bounds__(NT) void lupdate_kernel(const E *__restrict__ X, const E *__restrict__ P, int64_t n,
                                                     int64_t c1, int kc, E *__restrict__ T, int64_t ldt,
                                                     int64_t off) {
    typedef typename Frag<E>::type F;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t b = blockIdx.y, t0 = (int64_t)blockIdx.x * 64;
    if (wn >= (kc + 31) / 32) return;  // the kernel has no barrier
    const int64_t t = t0 + wm * 32 + lr;
    const int kk = wn * 32 + lr;
    const bool tok = t < n, kok = kk < kc;
    const E *pa = X + (b * n + (tok ? t : 0)) * c1;
    const E *pb = P + (b * kc + (kok ? kk : 0)) * c1;
    f32x16 acc = f32x16{};
#pragma unroll 4
    for (int64_t f = 0; f < c1; f += 16) {
        const F fa = tok ? ld_frag(pa + f + lk) : F{};
        const F fb = kok ? ld_frag(pb + f + lk) : F{};
        acc = mma16(acc, fa, fb);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int64_t row = t0 + wm * 32 + acc_row(lane, q);
        if (row < n && kok) T[(b * n + row) * ldt + off + kk] = to_elem<E>(acc[q]);
    }
}

}  // namespace

template <typename E>
hipError_t launch_als_lupdate(const AlsArgs<E> &a, int last, float alpha, hipStream_t st, const EventMark &mark) {
    if (a.B <= 0) return hipSuccess;
    if (a.kc < 16 || a.kc > 64 || a.kc % 16 != 0) return hipErrorInvalidValue;
    hipError_t e;
    hipLaunchKernelGGL((transpose_r1_kernel<E>), dim3((unsigned)((a.c2 + 63) / 64), (unsigned)a.B), dim3(NT), 0, st,
                       a.R1t, a.c2, a.kc, a.R1row);
    if ((e = mark(hipGetLastError())) != hipSuccess) return e;
    // S'^T = R' W_res^T: [B kc][c1]
    if ((e = mark(launch_gemm_store<E>(a.R1row, a.c2, a.Wres, a.c2, a.B * a.kc, a.c1, a.c2, a.Sp, a.c1, st))) !=
        hipSuccess)
        return e;
    hipLaunchKernelGGL((gram_rows_kernel<E>), dim3((unsigned)a.B), dim3(NT), 0, st, a.R1row, a.c2, a.kc, a.H);
    if ((e = mark(hipGetLastError())) != hipSuccess) return e;
    hipLaunchKernelGGL(als_coef_kernel, dim3((unsigned)a.B), dim3(NT), 0, st, a.H, a.C, a.kc, a.k_real, a.lambda,
                       last, alpha, a.Kp, a.flags);
    if ((e = mark(hipGetLastError())) != hipSuccess) return e;
    const dim3 ga((unsigned)((a.c1 + NT - 1) / NT), (unsigned)a.B);
    switch (a.kc) {
    case 16: hipLaunchKernelGGL((als_apply_kernel<E, 16>), ga, dim3(NT), 0, st, a.Kp, a.Sp, a.c1, a.P); break;
    case 32: hipLaunchKernelGGL((als_apply_kernel<E, 32>), ga, dim3(NT), 0, st, a.Kp, a.Sp, a.c1, a.P); break;
    case 48: hipLaunchKernelGGL((als_apply_kernel<E, 48>), ga, dim3(NT), 0, st, a.Kp, a.Sp, a.c1, a.P); break;
    default: hipLaunchKernelGGL((als_apply_kernel<E, 64>), ga, dim3(NT), 0, st, a.Kp, a.Sp, a.c1, a.P); break;
    }
    if ((e = mark(hipGetLastError())) != hipSuccess) return e;
    hipLaunchKernelGGL((lupdate_kernel<E>), dim3((unsigned)((a.n + 63) / 64), (unsigned)a.B), dim3(NT), 0, st, a.X,
                       a.P, a.n, a.c1, a.kc, a.T, a.ldt, a.off);
    return mark(hipGetLastError());
}

template hipError_t launch_als_lupdate<bf16>(const AlsArgs<bf16> &, int, float, hipStream_t, const EventMark &);
template hipError_t launch_als_lupdate<float>(const AlsArgs<float> &, int, float, hipStream_t, const EventMark &);

}  // namespace dyra
