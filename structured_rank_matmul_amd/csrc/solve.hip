// Per-instance right-factor statistics of the DyRA correction (gfx950).
//
// "DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
// DNNs", Eq. 5 / Algorithm 1 line 12:
//     R1_b = (L1_b^T L1_b + lambda I)^-1 (L1_b^T X_b) W_res
// and the output needs only the product L1_b R1_b.  With the Cholesky factor
// G = L1_b^T L1_b + lambda I = C C^T (§2.4 solves this SPD system per
// instance) the projector splits symmetrically,
//     L1_b G^-1 L1_b^T = Q_b Q_b^T,   Q_b = L1_b C^-T   (n x k),
// so the path carries Q_b in place of L1_b and R1 = (Q_b^T X_b) W_res.  The
// product is the same as Eq. 5's; Q_b is well scaled (orthonormal columns for
// lambda = 0), so rounding it and Q_b^T X_b to bf16 is not amplified by the
// conditioning of L1_b as the normal-equation form would be.
//
//   gram_q   one workgroup per instance: G (MFMA over tokens), Cholesky and the
//            triangular inverse C^-1 with the 64 x 64 matrix held in registers
//            (16 entries per thread, one barrier per column), then
//            Q_b^T = C^-1 L1_b^T by float32 MFMA, written token-contiguous (Qt)
//            and row-major over L1_b.
//   mprime   workgroup (instance b, 256 input features): M'_b = Q_b^T X_b.
#include "dyra_kernels.h"

#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;
constexpr int TK = 32;  // tokens per slice of the token contraction

// Optional per-phase timestamps for profiling builds (empty in the library).
#ifndef DYRA_PHASE_MARK
#define DYRA_PHASE_MARK(i)
#endif

__device__ __forceinline__ f32x8 frag_f32(const bf16 *p) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
    f32x8 r;
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] = (float)v[q];
    return r;
}
__device__ __forceinline__ f32x8 frag_f32(const float *p) { return ld_frag(p); }

// Transposes a [TK tokens][kc] slice of a row-major [tokens][kc] matrix into
// LDS dst[feature][token] (row stride ST); tokens at or beyond `tokens` read 0.
// Consecutive threads take consecutive tokens so the 16-bit LDS writes of a
// wavefront land in consecutive words.
template <typename E, int ST>
__device__ __forceinline__ void load_transposed(const E *src, int64_t ld, int64_t t0, int64_t tokens, int64_t col0,
                                                int64_t cols_valid, int cols, E *dst, int tid) {
    constexpr int VEC = Lay<E>::VEC;
    const int chunks = TK * (cols / VEC);
    for (int c = tid; c < chunks; c += NT) {
        const int tok = c % TK;
        const int j0 = (c / TK) * VEC;
        union { uint4 u; E e[VEC]; } v;
        v.u = (t0 + tok < tokens && col0 + j0 < cols_valid)
                  ? *reinterpret_cast<const uint4 *>(src + (t0 + tok) * ld + col0 + j0)
                  : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < VEC; ++q) dst[(j0 + q) * ST + tok] = v.e[q];
    }
}

// The k x k solve runs in float32 for bf16 data and in float64 for float32
// data (the float32 path is held to a 1e-5 relative error, which a float32
// Gram matrix cannot give when L1_b is ill-conditioned).
template <typename E> struct SolveT { typedef float type; };
template <> struct SolveT<float> { typedef double type; };

template <typename E>
__global__ __launch_bounds__(NT) void gram_q_kernel(E *__restrict__ L1, int64_t n, int64_t npad, int kc_real, int kc,
                                                    float lambda, E *__restrict__ Qt, int *__restrict__ flags) {
    typedef typename SolveT<E>::type AT;
    constexpr bool kMfma = sizeof(E) == 2;  // bf16: Gram and Q on MFMA; float32: float64 FMA
    constexpr int ST = TK + Lay<E>::PAD;
    constexpr int GS = 68;  // row stride of the LDS matrix (16-byte aligned rows)
    __shared__ __align__(16) E Lt[64 * ST];
    __shared__ __align__(16) AT G[64 * GS];
    __shared__ AT vec[2][64];
    __shared__ AT rowv[2][64];
    __shared__ int fail;
    __shared__ AT thresh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int j = tid & 63, i0 = tid >> 6;  // this thread owns entries (i0 + 4q, j), q = 0..15
    const int64_t b = blockIdx.x;
    E *Lb = L1 + b * n * kc;
    DYRA_PHASE_MARK(0);

    for (int e = tid; e < 64 * GS; e += NT) G[e] = AT(0);
    if (tid == 0) fail = 0;
    AT g[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) g[q] = AT(0);
    // ---- Gram matrix G = L1_b^T L1_b over the instance's tokens
    if constexpr (kMfma) {
        const int wm = wave >> 1, wn = wave & 1;
        const bool active = wm * 32 < kc && wn * 32 < kc;
        for (int e = tid; e < 64 * ST; e += NT) Lt[e] = to_elem<E>(0.f);
        __syncthreads();
        f32x16 acc = f32x16{};
        for (int64_t t0 = 0; t0 < n; t0 += TK) {
            load_transposed<E, ST>(Lb, kc, t0, n, 0, kc, kc, Lt, tid);
            __syncthreads();
            if (active) {
#pragma unroll
                for (int kk = 0; kk < TK; kk += 16)
                    acc = mma16(acc, ld_frag(Lt + (wm * 32 + lr) * ST + kk + lk),
                                ld_frag(Lt + (wn * 32 + lr) * ST + kk + lk));
            }
            __syncthreads();
        }
        if (active) {
#pragma unroll
            for (int t = 0; t < 16; ++t) G[(wm * 32 + acc_row(lane, t)) * GS + wn * 32 + lr] = acc[t];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) g[q] = G[(i0 + 4 * q) * GS + j];
    } else {
        // token slices staged row-major in Lt ([token][feature], row stride 64)
        for (int64_t t0 = 0; t0 < n; t0 += TK) {
            __syncthreads();
            for (int e = tid; e < TK * 64; e += NT) {
                const int t = e >> 6, c = e & 63;
                Lt[t * 64 + c] = (t0 + t < n && c < kc) ? Lb[(t0 + t) * kc + c] : to_elem<E>(0.f);
            }
            __syncthreads();
            const int tc = (int)((n - t0) < TK ? (n - t0) : TK);
            for (int t = 0; t < tc; ++t) {
                const AT lj = (AT)to_f32(Lt[t * 64 + j]);
#pragma unroll
                for (int q = 0; q < 16; ++q) g[q] += (AT)to_f32(Lt[t * 64 + i0 + 4 * q]) * lj;
            }
        }
    }
    // ---- G + lambda I on the real indices, identity on the padding
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int i = i0 + 4 * q;
        if (i < kc_real && j < kc_real) g[q] += (i == j) ? (AT)lambda : AT(0);
        else g[q] = (i == j) ? AT(1) : AT(0);
    }
    // a pivot below the working precision times the largest diagonal means a
    // numerically singular Gram matrix (possible only for lambda = 0)
#pragma unroll
    for (int q = 0; q < 16; ++q)
        if (i0 + 4 * q == j) vec[0][j] = g[q];  // the diagonal, one owner per entry
    __syncthreads();
    DYRA_PHASE_MARK(1);
    if (tid == 0) {
        AT dmax = AT(0);
        for (int i = 0; i < kc; ++i) dmax = dmax > vec[0][i] ? dmax : vec[0][i];
        const AT eps = sizeof(AT) == 4 ? AT(1.2e-7) : AT(2.3e-16);
        thresh = lambda > 0.f ? AT(0) : (AT)kc * eps * dmax;
        if (!(dmax > AT(0))) fail = 1;
    }
    __syncthreads();
    const AT th = thresh;
    // ---- Cholesky G = C C^T (lower), right-looking, one barrier per column, no branches
    for (int k = 0; k < kc; ++k) {
        AT *colk = vec[k & 1];
        if (j == k) {
#pragma unroll
            for (int q = 0; q < 16; ++q) colk[i0 + 4 * q] = g[q];
        }
        __syncthreads();
        AT pk = colk[k];
        if (!(pk > th)) {
            if (tid == 0) fail = 1;
            pk = AT(1);
        }
        const AT d = sqrt(pk), dinv = AT(1) / d, rinv = dinv * dinv;
        const AT cjr = colk[j] * rinv;
        const bool jact = j >= k && j < kc;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = i0 + 4 * q;
            const AT ci = colk[i];
            const AT col = (i == k) ? d : ci * dinv;
            const AT upd = g[q] - ci * cjr;
            const AT v = (j == k) ? col : ((j <= i) ? upd : g[q]);
            g[q] = (jact && i >= k && i < kc) ? v : g[q];
        }
    }
    // upper part to zero: g now holds C
#pragma unroll
    for (int q = 0; q < 16; ++q) g[q] = (j > i0 + 4 * q) ? AT(0) : g[q];
    __syncthreads();
    DYRA_PHASE_MARK(2);
    // ---- C^-1 by in-place Gauss-Jordan (stays lower-triangular), no branches
    for (int k = 0; k < kc; ++k) {
        AT *colk = vec[k & 1];
        AT *rowk = rowv[k & 1];
        if (j == k) {
#pragma unroll
            for (int q = 0; q < 16; ++q) colk[i0 + 4 * q] = g[q];
        }
        if ((k & 3) == i0) {
            // g[k >> 2] without a runtime register index (which would go to scratch)
            AT v = AT(0);
#pragma unroll
            for (int q = 0; q < 16; ++q) v = (q == (k >> 2)) ? g[q] : v;
            rowk[j] = v;
        }
        __syncthreads();
        const AT inv = AT(1) / rowk[k];
        const AT rji = rowk[j] * inv;
        const bool jin = j < kc;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = i0 + 4 * q;
            const AT ci = colk[i];
            const AT vk = (j == k) ? inv : rji;
            const AT v = (i == k) ? vk : ((j == k) ? -ci * inv : g[q] - ci * rji);
            g[q] = (jin && i < kc) ? v : g[q];
        }
    }
    __syncthreads();
    DYRA_PHASE_MARK(3);
    const bool failed = fail != 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) G[(i0 + 4 * q) * GS + j] = failed ? AT(0) : g[q];
    __syncthreads();
    // ---- Q^T = C^-1 L1_b^T -> Qt[b] (token-contiguous) and Q in place of L1_b
    E *Qb = Qt + b * kc * npad;
    if constexpr (kMfma) {
        const int nrb = (kc + 31) / 32;
        for (int64_t tb = wave; tb * 32 < npad; tb += 4) {
            const int64_t t = tb * 32 + lr;
            f32x16 z[2] = {f32x16{}, f32x16{}};
            for (int kk = 0; kk < kc; kk += 16) {
                const f32x8 fb = t < n ? frag_f32(Lb + t * kc + kk + lk) : f32x8{};
                for (int ib = 0; ib < nrb; ++ib)
                    z[ib] = mma16(z[ib], ld_frag((const float *)&G[(ib * 32 + lr) * GS + kk + lk]), fb);
            }
            for (int ib = 0; ib < nrb; ++ib) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int i = ib * 32 + acc_row(lane, q);
                    if (i < kc) Qb[(int64_t)i * npad + t] = to_elem<E>(z[ib][q]);
                }
                if (t < n) {
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        const int i = ib * 32 + acc_row(lane, 4 * gg);
                        if (i >= kc) continue;
#pragma unroll
                        for (int q = 0; q < 4; ++q) Lb[t * kc + i + q] = to_elem<E>(z[ib][4 * gg + q]);
                    }
                }
            }
        }
    } else {
        // one token per thread: q_t = C^-1 l_t in float64
        for (int64_t t = tid; t < npad; t += NT) {
            AT l[64];
#pragma unroll
            for (int c = 0; c < 64; ++c) l[c] = (t < n && c < kc) ? (AT)to_f32(Lb[t * kc + c]) : AT(0);
            for (int i = 0; i < kc; ++i) {
                AT sum = AT(0);
#pragma unroll
                for (int c = 0; c < 64; ++c) sum += G[i * GS + c] * l[c];
                Qb[(int64_t)i * npad + t] = to_elem<E>((float)sum);
                if (t < n) Lb[t * kc + i] = to_elem<E>((float)sum);
            }
        }
    }
    DYRA_PHASE_MARK(4);
    if (tid == 0) flags[b] = failed ? 1 : 0;
}

template <typename E>
__global__ __launch_bounds__(NT) void mprime_kernel(const E *__restrict__ X, const E *__restrict__ Qt, int64_t n,
                                                    int64_t npad, int64_t c1, int kc, E *__restrict__ Mp) {
    constexpr int CW = 256;
    constexpr int ST = TK + Lay<E>::PAD;
    __shared__ __align__(16) E Xt[CW * ST];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int64_t b = blockIdx.y;
    const int64_t col0 = (int64_t)blockIdx.x * CW;
    const E *Xb = X + b * n * c1;
    const E *Zb = Qt + b * kc * npad;
    const int nrb = (kc + 31) / 32;
    typedef typename Frag<E>::type F;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    for (int64_t t0 = 0; t0 < n; t0 += TK) {
        load_transposed<E, ST>(Xb, c1, t0, n, col0, c1, CW, Xt, tid);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; kk += 16) {
            F fa[2], fb[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int i = ib * 32 + lr;
                fa[ib] = (ib < nrb && i < kc) ? ld_frag(Zb + (int64_t)i * npad + t0 + kk + lk) : F{};
            }
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) fb[jb] = ld_frag(Xt + (wave * 64 + jb * 32 + lr) * ST + kk + lk);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
                if (ib < nrb)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = mma16(acc[ib][jb], fa[ib], fb[jb]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        if (ib >= nrb) continue;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int64_t col = col0 + wave * 64 + jb * 32 + lr;
            if (col >= c1) continue;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int i = ib * 32 + acc_row(lane, q);
                if (i < kc) Mp[(b * kc + i) * c1 + col] = to_elem<E>(acc[ib][jb][q]);
            }
        }
    }
}

}  // namespace

template <typename E>
hipError_t launch_gram_q(E *L1, int64_t B, int64_t n, int64_t npad, int kc_real, int kc, float lambda, E *Qt,
                         int *flags, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL((gram_q_kernel<E>), dim3((unsigned)B), dim3(NT), 0, st, L1, n, npad, kc_real, kc, lambda, Qt,
                       flags);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_mprime(const E *X, const E *Qt, int64_t B, int64_t n, int64_t npad, int64_t c1, int kc, E *Mp,
                         hipStream_t st) {
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL((mprime_kernel<E>), dim3((unsigned)((c1 + 255) / 256), (unsigned)B), dim3(NT), 0, st, X, Qt,
                       n, npad, c1, kc, Mp);
    return hipGetLastError();
}

template hipError_t launch_gram_q<bf16>(bf16 *, int64_t, int64_t, int64_t, int, int, float, bf16 *, int *,
                                        hipStream_t);
template hipError_t launch_gram_q<float>(float *, int64_t, int64_t, int64_t, int, int, float, float *, int *,
                                         hipStream_t);
template hipError_t launch_mprime<bf16>(const bf16 *, const bf16 *, int64_t, int64_t, int64_t, int64_t, int, bf16 *,
                                        hipStream_t);
template hipError_t launch_mprime<float>(const float *, const float *, int64_t, int64_t, int64_t, int64_t, int,
                                         float *, hipStream_t);

}  // namespace dyra
