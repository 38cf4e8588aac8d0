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
// K' = Z^-1 C^T (or alpha Z^-1 for the last update) per instance, and
// L_new = (X_b S'_b) K'_b into the L columns of the left-pass buffer.
#include "dyra_kernels.h"

#include "elim.h"
#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;

// R1row[b][kk][c] = R1t[b][c][kk]; 64 columns c per workgroup through LDS,
// 16-byte loads along kk and 16-byte stores along c.
template <typename E>
__global__ __launch_bounds__(NT) void transpose_r1_kernel(const E *__restrict__ R1t, int64_t c2, int kc,
                                                          E *__restrict__ R1row) {
    constexpr int V = 16 / (int)sizeof(E);
    __shared__ __align__(16) E tile[64][64 + V];  // [c][kk]; rows stay 16-byte aligned
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y, c0 = (int64_t)blockIdx.x * 64;
    const int cw = c2 - c0 < 64 ? (int)(c2 - c0) : 64;  // 32 or 64 (c2 is a multiple of 32)
    const E *src = R1t + (b * c2 + c0) * kc;
    const int vpr = kc / V;
    for (int e = tid; e < cw * vpr; e += NT) {
        const int c = e / vpr, v = e - c * vpr;
        *reinterpret_cast<uint4 *>(&tile[c][v * V]) = *reinterpret_cast<const uint4 *>(src + (int64_t)c * kc + v * V);
    }
    __syncthreads();
    const int vpc = cw / V;
    for (int e = tid; e < kc * vpc; e += NT) {
        const int kk = e / vpc, v = e - kk * vpc;
        union { uint4 u; E x[V]; } w;
#pragma unroll
        for (int q = 0; q < V; ++q) w.x[q] = tile[v * V + q][kk];
        *reinterpret_cast<uint4 *>(R1row + (b * kc + kk) * c2 + c0 + v * V) = w.u;
    }
}

// Partial Gram matrices of R'_b: Hp[s][b] = sum over the s-th of
// kAlsGramSplit column ranges of R'_b R'_b^T ([kc][kc] float32; summed by
// als_coef_kernel).  Grid (B, kAlsGramSplit); each wavefront takes a quarter
// of its workgroup's range and all (up to 2 x 2) 32 x 32 blocks, fragments
// prefetched four steps ahead; the four partials are added from LDS.
template <typename E>
__global__ __launch_bounds__(NT) void gram_rows_kernel(const E *__restrict__ R1row, int64_t c2, int kc,
                                                       float *__restrict__ Hp) {
    typedef typename Frag<E>::type F;
    constexpr int U = 4;
    __shared__ float red[4][64][65];  // one partial per wavefront
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int64_t b = blockIdx.x, B = gridDim.x;
    const int sp = blockIdx.y;
    const int nb = (kc + 31) / 32;
    const int64_t steps = c2 / 16;
    const int part = sp * 4 + wave, parts = kAlsGramSplit * 4;
    const int64_t s0 = steps * part / parts, s1 = steps * (part + 1) / parts;
    const bool ok0 = lr < kc, ok1 = 32 + lr < kc;
    const E *p0 = R1row + (b * kc + (ok0 ? lr : 0)) * c2 + lk;
    const E *p1 = R1row + (b * kc + (ok1 ? 32 + lr : 0)) * c2 + lk;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    F f0[U], f1[U];
    auto load = [&](int64_t t, F (&x0)[U], F (&x1)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = t + u < s1;
            x0[u] = (ok0 && in) ? ld_frag(p0 + (t + u) * 16) : F{};
            x1[u] = (ok1 && in) ? ld_frag(p1 + (t + u) * 16) : F{};
        }
    };
    load(s0, f0, f1);
    for (int64_t t = s0; t < s1; t += U) {
        F n0[U], n1[U];
        load(t + U, n0, n1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc[0][0] = mma16(acc[0][0], f0[u], f0[u]);
            if (nb > 1) {
                acc[0][1] = mma16(acc[0][1], f0[u], f1[u]);
                acc[1][0] = mma16(acc[1][0], f1[u], f0[u]);
                acc[1][1] = mma16(acc[1][1], f1[u], f1[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            f0[u] = n0[u];
            f1[u] = n1[u];
        }
    }
    // (float atomics on LDS cost several times the whole Gram here)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (i < nb && j < nb)
#pragma unroll
                for (int q = 0; q < 16; ++q) red[wave][i * 32 + acc_row(lane, q)][j * 32 + lr] = acc[i][j][q];
    __syncthreads();
    float *H = Hp + ((int64_t)sp * B + b) * kc * kc;
    for (int e = tid; e < kc * kc; e += NT) {
        const int i = e / kc, j = e - i * kc;
        H[e] = (red[0][i][j] + red[1][i][j]) + (red[2][i][j] + red[3][i][j]);
    }
}

// K'_b ([kc][kc] float32) from H'_b (sum of the kAlsGramSplit partials) and
// C_b, in float64:
//   Z = H' + lambda C^T C on the real indices (identity on the padding),
//   K' = Z^-1 C^T (the L update is followed by an R update: rows of P are
//   then the columns of L_new = X S' K'), or alpha Z^-1 (the last update:
//   L_new R = X S' Z^-1 R', alpha weighting the correction),
// by Gauss-Jordan elimination of [Z | C^T] (or [Z | alpha I]); Z is SPD, so
// no pivoting is needed and its pivots are those of Z = D D^T squared.
// Thread (c, i1) holds column c of the 64 x 128 augmented matrix for rows
// i1, i1 + 2, ..., in registers; step K publishes pivot row K and column K
// through LDS.  A pivot at or below kc times float32 precision times Z's
// largest diagonal entry (possible only for lambda = 0, when R' is rank
// deficient) sets flags[b] and makes K' zero: the instance then gets no
// correction.
__global__ __launch_bounds__(NT) void als_coef_kernel(const float *__restrict__ Hp, const double *__restrict__ C,
                                                      int kc, int kc_real, float lambda, int last, float alpha,
                                                      float *__restrict__ Kp, int *__restrict__ flags) {
    __shared__ double A[64][129];  // [Z | right-hand side], formed here, then held in registers
    __shared__ double Cs[64][65];
    __shared__ double rowK[128], colK[64];
    __shared__ int fail;
    __shared__ double thresh;
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x, B = gridDim.x;
    for (int e = tid; e < 64 * 64; e += NT) {
        const int i = e >> 6, j = e & 63;
        Cs[i][j] = (i < kc && j < kc) ? C[b * kc * kc + i * kc + j] : 0.0;
    }
    if (tid == 0) fail = 0;
    __syncthreads();
    {
        // thread (i0, j) forms entries (i0 + 4 q, j), q = 0..15
        const int j = tid & 63, i0 = tid >> 6;
        double s[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) s[q] = 0.0;
        if (lambda > 0.f) {
            for (int m = 0; m < kc; ++m) {
                const double cmj = Cs[m][j];
#pragma unroll
                for (int q = 0; q < 16; ++q) s[q] += Cs[m][i0 + 4 * q] * cmj;
            }
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = i0 + 4 * q;
            double z = 0.0, rhs = 0.0;
            if (i < kc && j < kc) {
                if (i < kc_real && j < kc_real) {
                    float h = 0.f;
                    for (int p = 0; p < kAlsGramSplit; ++p) h += Hp[(((int64_t)p * B + b) * kc + i) * kc + j];
                    z = (double)h + (double)lambda * s[q];
                } else {
                    z = i == j ? 1.0 : 0.0;
                }
                rhs = last ? (i == j ? (double)alpha : 0.0) : Cs[j][i];
            }
            A[i][j] = z;
            A[i][64 + j] = rhs;
        }
    }
    __syncthreads();
    if (tid == 0) {
        double dmax = 0.0;
        for (int i = 0; i < kc_real; ++i) dmax = A[i][i] > dmax ? A[i][i] : dmax;
        thresh = lambda > 0.f ? 0.0 : (double)kc * 1.2e-7 * dmax;
        if (!(dmax > 0.0)) fail = 1;
    }
    const int c = tid & 127, i1 = tid >> 7;  // i1 is uniform over each wavefront
    double a[32];
#pragma unroll
    for (int q = 0; q < 32; ++q) a[q] = A[i1 + 2 * q][c];
    __syncthreads();
    const double th = thresh;
    for (int K = 0; K < kc; ++K) {
        if (i1 == (K & 1)) {
#pragma unroll
            for (int q = 0; q < 32; ++q)
                if (q == (K >> 1)) rowK[c] = a[q];
        }
        if (c == K) {
#pragma unroll
            for (int q = 0; q < 32; ++q) colK[i1 + 2 * q] = a[q];
        }
        __syncthreads();
        double pk = rowK[K];
        const bool bad = K < kc_real && !(pk > th);
        if (bad) pk = 1.0;
        if (bad && tid == 0) fail = 1;
        const double rk = rowK[c] / pk;
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            const int i = i1 + 2 * q;
            a[q] = (i == K) ? rk : a[q] - colK[i] * rk;
        }
        __syncthreads();
    }
    const bool failed = fail != 0;
    if (c >= 64 && c - 64 < kc) {
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            const int i = i1 + 2 * q;
            if (i < kc) Kp[b * kc * kc + (int64_t)i * kc + (c - 64)] = failed ? 0.f : (float)a[q];
        }
    }
    if (tid == 0 && failed) flags[b] = 1;
}

// The same K'_b for bf16 plans, in float32 on one wavefront per instance with
// the lane-per-row elimination of elim.h (no barrier, no LDS round trip per
// pivot): lane i holds row i of Z and row i of RHS^T (alpha I or C).
// Eliminating [Z; RHS^T] leaves the Cholesky factor D of Z in g and
// U = RHS^T D^-T in u; back substitution gives u = U D^-1 = RHS^T Z^-1, row i
// of K'^T, i.e. column i of K' = Z^-1 RHS.  Same breakdown rule as above.
template <int KC>
__global__ __launch_bounds__(64) void als_coef32_kernel(const float *__restrict__ Hp, const double *__restrict__ C,
                                                        int kc_real, float lambda, int last, float alpha,
                                                        float *__restrict__ Kp, int *__restrict__ flags) {
    __shared__ float Cs[KC][KC + 1];
    __shared__ float Zs[64][KC + 1];
    const int i = threadIdx.x;  // the row this lane holds
    const int64_t b = blockIdx.x, B = gridDim.x;
    for (int e = i; e < KC * KC; e += 64) Cs[e / KC][e % KC] = (float)C[b * KC * KC + e];
    __syncthreads();
    // Z formed in LDS by the whole wavefront (consecutive lanes on consecutive
    // entries, the partial sums' loads independent), then row i into registers
#pragma unroll 4
    for (int e = i; e < KC * KC; e += 64) {
        const int r = e / KC, c = e - r * KC;
        float z;
        if (r < kc_real && c < kc_real) {
            float h = 0.f;
#pragma unroll
            for (int p = 0; p < kAlsGramSplit; ++p) h += Hp[((int64_t)p * B + b) * KC * KC + e];
            float s = 0.f;
            if (lambda > 0.f)
                for (int m = 0; m < KC; ++m) s = fmaf(Cs[m][r], Cs[m][c], s);
            z = fmaf(lambda, s, h);
        } else {
            z = r == c ? 1.f : 0.f;
        }
        Zs[r][c] = z;
    }
    for (int e = i; e < (64 - KC) * KC; e += 64) Zs[KC + e / KC][e % KC] = 0.f;  // lanes past KC hold no row
    __syncthreads();
    float g[KC], u[KC];
    float diag = 0.f;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        const float z = Zs[i][j];
        g[j] = z;
        u[j] = i < KC ? (last ? (i == j ? alpha : 0.f) : Cs[i][j]) : 0.f;
        diag = (i == j && i < kc_real) ? z : diag;
    }
    float dmax = diag;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dmax = fmaxf(dmax, __shfl_xor(dmax, o));
    const float th = lambda > 0.f ? 0.f : (float)KC * 1.2e-7f * dmax;
    bool fail = !(dmax > 0.f);
    elim_step<KC, 0>(g, u, kc_real, th, fail);
    back_step<KC, KC - 1>(g, u);
    if (i < KC) {
#pragma unroll
        for (int j = 0; j < KC; ++j) Kp[(b * KC + j) * KC + i] = fail ? 0.f : u[j];
    }
    if (i == 0 && fail) flags[b] = 1;
}

// The new L of instance b into the L columns of the left-pass buffer:
//   T[b*n + t][off + kk] = sum_j (X_b S'_b)[t][j] K'_b[j][kk],
// with S'_b stored by rows (Sp[b*kc + j][f] = S'[f][j]).  Workgroup (64
// tokens, instance b); each wavefront takes one 32 x 32 block of X_b S'_b,
// fragments straight from global memory with the next U steps prefetched
// while the current U are multiplied; the 64 x kc block then meets K'_b in
// LDS and each lane forms its outputs in float32 (one rounding, at the store).
template <typename E>
__global__ __launch_bounds__(NT) void lupdate_kernel(const E *__restrict__ X, const E *__restrict__ Sp,
                                                     const float *__restrict__ Kp, int64_t n, int64_t c1, int kc,
                                                     E *__restrict__ T, int64_t ldt, int64_t off) {
    typedef typename Frag<E>::type F;
    constexpr int U = sizeof(E) == 2 ? 8 : 4;
    __shared__ float Ys[64][65];  // (X_b S'_b)[token][j]
    __shared__ float Ks[64][65];  // K'_b[j][kk]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t b = blockIdx.y, t0 = (int64_t)blockIdx.x * 64;
    for (int e = tid; e < 64 * 64; e += NT) {
        const int j = e >> 6, kk = e & 63;
        Ks[j][kk] = (j < kc && kk < kc) ? Kp[(b * kc + j) * kc + kk] : 0.f;
    }
    const bool active = wn < (kc + 31) / 32;  // waves past the correction width only join the barrier
    const int64_t t = t0 + wm * 32 + lr;
    const int jj = wn * 32 + lr;
    const bool tok = t < n, jok = active && jj < kc;
    const E *pa = X + (b * n + (tok ? t : 0)) * c1 + lk;
    const E *pb = Sp + (b * kc + (jok ? jj : 0)) * c1 + lk;
    f32x16 acc = f32x16{};
    if (active) {
        F fa[U], fb[U];
        auto load = [&](int64_t f0, F (&xa)[U], F (&xb)[U]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t f = f0 + 16 * u;
                const bool in = f < c1;
                xa[u] = (tok && in) ? ld_frag(pa + f) : F{};
                xb[u] = (jok && in) ? ld_frag(pb + f) : F{};
            }
        };
        load(0, fa, fb);
        for (int64_t f0 = 0; f0 < c1; f0 += 16 * U) {
            F na[U], nb[U];
            load(f0 + 16 * U, na, nb);
#pragma unroll
            for (int u = 0; u < U; ++u) acc = mma16(acc, fa[u], fb[u]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                fa[u] = na[u];
                fb[u] = nb[u];
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) Ys[wm * 32 + acc_row(lane, q)][jj] = acc[q];  // zero where !jok
    __syncthreads();
    if (!active) return;  // no barrier follows
    const int kk = wn * 32 + lr;
    if (kk >= kc) return;
#pragma unroll 4
    for (int q = 0; q < 16; ++q) {
        const int r = wm * 32 + acc_row(lane, q);
        const int64_t row = t0 + r;
        float v = 0.f;
        for (int j = 0; j < kc; ++j) v = fmaf(Ys[r][j], Ks[j][kk], v);
        if (row < n) T[(b * n + row) * ldt + off + kk] = to_elem<E>(v);
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
    hipLaunchKernelGGL((gram_rows_kernel<E>), dim3((unsigned)a.B, kAlsGramSplit), dim3(NT), 0, st, a.R1row, a.c2,
                       a.kc, a.H);
    if ((e = mark(hipGetLastError())) != hipSuccess) return e;
    if constexpr (sizeof(E) == 2) {
        const dim3 g1((unsigned)a.B);
        switch (a.kc) {
        case 16: hipLaunchKernelGGL(als_coef32_kernel<16>, g1, dim3(64), 0, st, a.H, a.C, a.k_real, a.lambda, last, alpha, a.Kp, a.flags); break;
        case 32: hipLaunchKernelGGL(als_coef32_kernel<32>, g1, dim3(64), 0, st, a.H, a.C, a.k_real, a.lambda, last, alpha, a.Kp, a.flags); break;
        case 48: hipLaunchKernelGGL(als_coef32_kernel<48>, g1, dim3(64), 0, st, a.H, a.C, a.k_real, a.lambda, last, alpha, a.Kp, a.flags); break;
        default: hipLaunchKernelGGL(als_coef32_kernel<64>, g1, dim3(64), 0, st, a.H, a.C, a.k_real, a.lambda, last, alpha, a.Kp, a.flags); break;
        }
    } else {
        // float32 plans keep float64 for Z^-1 (their parity bar is 1e-5)
        hipLaunchKernelGGL(als_coef_kernel, dim3((unsigned)a.B), dim3(NT), 0, st, a.H, a.C, a.kc, a.k_real, a.lambda,
                           last, alpha, a.Kp, a.flags);
    }
    if ((e = mark(hipGetLastError())) != hipSuccess) return e;
    hipLaunchKernelGGL((lupdate_kernel<E>), dim3((unsigned)((a.n + 63) / 64), (unsigned)a.B), dim3(NT), 0, st, a.X,
                       a.Sp, a.Kp, a.n, a.c1, a.kc, a.T, a.ldt, a.off);
    return mark(hipGetLastError());
}

template hipError_t launch_als_lupdate<bf16>(const AlsArgs<bf16> &, int, float, hipStream_t, const EventMark &);
template hipError_t launch_als_lupdate<float>(const AlsArgs<float> &, int, float, hipStream_t, const EventMark &);

}  // namespace dyra
