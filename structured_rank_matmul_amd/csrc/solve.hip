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
// L1_b lives in columns [off, off + kc) of the rows b*n .. b*n + n - 1 of the
// row-major pass output T (leading dimension ldt) and Q_b overwrites it there.
//
//   cholq (bf16)  workgroup (token block of 256, instance b): G by MFMA over
//            all n tokens of b, then every wavefront factors G with one matrix
//            row per lane and, in the same elimination steps, turns its 64
//            token rows of L1_b into rows of Q_b: factoring [G; L1_b] leaves
//            L1_b C^-T in the lower block.  The pivot row's entries reach all
//            lanes through v_readlane, so the factorisation has no barrier and
//            no LDS traffic.
//   gram_q (float32)  one workgroup per instance, all in float64: G, a
//            right-looking Cholesky and the inverse C^-1 with 16 matrix entries
//            per thread, then q_t = C^-1 l_t per token.
//   mprime   workgroup (instance b, 256 input features): M'_b = Q_b^T X_b.
#include "dyra_kernels.h"

#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;
constexpr int TK = 32;  // tokens per slice of the token contraction (mprime)

// Optional per-phase timestamps for profiling builds (empty in the library).
#ifndef DYRA_PHASE_MARK
#define DYRA_PHASE_MARK(i)
#endif

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

__device__ __forceinline__ float bcast(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---------------------------------------------------------------- bf16 path
template <int KC>
__global__ __launch_bounds__(NT) void cholq_kernel(bf16 *__restrict__ T, int64_t ldt, int64_t off, int64_t n,
                                                   int64_t npad, int kc_real, float lambda, bf16 *__restrict__ Qt,
                                                   int *__restrict__ flags) {
    constexpr int GS = 68;        // row stride (floats) of G in LDS
    constexpr int TT = 64;        // tokens per Gram chunk
    constexpr int ST = TT + 8;    // row stride (bf16) of the transposed chunk
    constexpr int NBLK = (KC + 31) / 32;
    __shared__ __align__(16) bf16 Lt[64 * ST];
    __shared__ __align__(16) float Gs[64 * GS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int64_t b = blockIdx.y;
    bf16 *const Tb = T + b * n * ldt + off;  // token t of instance b: Tb + t * ldt
    DYRA_PHASE_MARK(0);

    // ---- G = L1_b^T L1_b over all n tokens, 32x32 blocks on MFMA
    const int wm = wave >> 1, wn = wave & 1;
    const bool gact = wm < NBLK && wn < NBLK;
    f32x16 acc = f32x16{};
    uint4 reg[2];
    // chunk of TT tokens x 64 features: thread c = tid + 256 p loads token
    // c % 64, features 8 (c / 64) .. +7 (features >= KC and tokens >= n read 0)
    auto gload = [&](int64_t t0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int c = tid + p * NT;
            const int tok = c & 63, j0 = (c >> 6) * 8;
            const bool ok = t0 + tok < n && j0 < KC;
            const uint4 v = *reinterpret_cast<const uint4 *>(Tb + (ok ? (t0 + tok) * ldt + j0 : 0));
            reg[p] = ok ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto gstore = [&]() {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int c = tid + p * NT;
            const int tok = c & 63, j0 = (c >> 6) * 8;
            union { uint4 u; bf16 e[8]; } v;
            v.u = reg[p];
#pragma unroll
            for (int q = 0; q < 8; ++q) Lt[(j0 + q) * ST + tok] = v.e[q];
        }
    };
    const int64_t nch = (n + TT - 1) / TT;
    gload(0);
    for (int64_t ch = 0; ch < nch; ++ch) {
        __syncthreads();
        gstore();
        __syncthreads();
        if (ch + 1 < nch) gload((ch + 1) * TT);
        if (gact) {
#pragma unroll
            for (int kk = 0; kk < TT; kk += 16)
                acc = mma16(acc, ld_frag(Lt + (wm * 32 + lr) * ST + kk + lk), ld_frag(Lt + (wn * 32 + lr) * ST + kk + lk));
        }
    }
    if (gact) {
#pragma unroll
        for (int t = 0; t < 16; ++t) Gs[(wm * 32 + acc_row(lane, t)) * GS + wn * 32 + lr] = acc[t];
    }
    __syncthreads();
    DYRA_PHASE_MARK(1);

    // ---- lane i holds row i of G + lambda I (identity rows past kc_real)
    const int i = lane;
    float g[KC];
#pragma unroll
    for (int m = 0; m < KC; m += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(&Gs[(i < KC ? i : 0) * GS + m]);
        g[m] = v.x; g[m + 1] = v.y; g[m + 2] = v.z; g[m + 3] = v.w;
    }
    const float diag = i < kc_real ? Gs[i * GS + i] : 0.f;
#pragma unroll
    for (int m = 0; m < KC; ++m) {
        const float e = (i < kc_real && m < kc_real) ? g[m] : 0.f;
        g[m] = (m == i) ? (i < kc_real ? e + lambda : 1.f) : e;
    }
    // a pivot at or below the working precision times the largest diagonal
    // marks a numerically singular G (possible only for lambda = 0)
    float dmax = diag;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dmax = fmaxf(dmax, __shfl_xor(dmax, o));
    const float th = lambda > 0.f ? 0.f : (float)KC * 1.2e-7f * dmax;
    bool fail = !(dmax > 0.f);

    // ---- this wavefront's 64 token rows of L1_b
    const int64_t t = (int64_t)blockIdx.x * NT + wave * 64 + lane;
    const bool tin = t < n;
    float l[KC];
#pragma unroll
    for (int m = 0; m < KC; m += 8) {
        union { uint4 u; bf16 e[8]; } v;
        v.u = *reinterpret_cast<const uint4 *>(Tb + (tin ? t * ldt : 0) + m);
#pragma unroll
        for (int q = 0; q < 8; ++q) l[m + q] = tin ? (float)v.e[q] : 0.f;
    }
    DYRA_PHASE_MARK(2);

    // ---- elimination: step k takes pivot row k (lane k) to all lanes
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        float pk = bcast(g[k], k);
        const bool bad = k < kc_real && !(pk > th);  // padding pivots are 1
        fail = fail || bad;
        pk = bad ? 1.f : pk;
        const float rp = 1.f / pk;
        const float a = g[k] * rp;      // G rows: C[i][k] / C[k][k]
        const float bt = l[k] * rp;     // token rows: Q[t][k] / C[k][k]
        l[k] = l[k] * (1.f / sqrtf(pk));
#pragma unroll
        for (int m = k + 1; m < KC; ++m) {
            const float s = bcast(g[m], k);   // trailing row k = C[m][k] C[k][k]
            g[m] = fmaf(-a, s, g[m]);
            l[m] = fmaf(-bt, s, l[m]);
        }
    }
    DYRA_PHASE_MARK(3);

    // ---- Q_b rows in place of L1_b, and Qt[b] = Q_b^T (token-contiguous, zero past n)
    if (tin) {
#pragma unroll
        for (int m = 0; m < KC; m += 8) {
            union { uint4 u; bf16 e[8]; } v;
#pragma unroll
            for (int q = 0; q < 8; ++q) v.e[q] = fail ? bf16(0.f) : (bf16)l[m + q];
            *reinterpret_cast<uint4 *>(Tb + t * ldt + m) = v.u;
        }
    }
    if (t < npad) {
        bf16 *qb = Qt + b * KC * npad + t;
#pragma unroll
        for (int m = 0; m < KC; ++m) qb[(int64_t)m * npad] = fail ? bf16(0.f) : (bf16)l[m];
    }
    if (blockIdx.x == 0 && tid == 0) flags[b] = fail ? 1 : 0;
    DYRA_PHASE_MARK(4);
}

// ------------------------------------------------------------- float32 path
__global__ __launch_bounds__(NT) void gram_q_f32_kernel(float *__restrict__ T, int64_t ldt, int64_t off, int64_t n,
                                                        int64_t npad, int kc_real, int kc, float lambda,
                                                        float *__restrict__ Qt, int *__restrict__ flags) {
    typedef double AT;
    constexpr int GS = 68;
    __shared__ __align__(16) float Lt[TK * 64];
    __shared__ __align__(16) AT G[64 * GS];
    __shared__ AT vec[2][64];
    __shared__ AT rowv[2][64];
    __shared__ int fail;
    __shared__ AT thresh;
    const int tid = threadIdx.x;
    const int j = tid & 63, i0 = tid >> 6;  // this thread owns entries (i0 + 4q, j), q = 0..15
    const int64_t b = blockIdx.x;
    float *Lb = T + b * n * ldt + off;

    if (tid == 0) fail = 0;
    AT g[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) g[q] = AT(0);
    // ---- G = L1_b^T L1_b, token slices staged row-major in Lt ([token][feature])
    for (int64_t t0 = 0; t0 < n; t0 += TK) {
        __syncthreads();
        for (int e = tid; e < TK * 64; e += NT) {
            const int tt = e >> 6, c = e & 63;
            Lt[tt * 64 + c] = (t0 + tt < n && c < kc) ? Lb[(t0 + tt) * ldt + c] : 0.f;
        }
        __syncthreads();
        const int tc = (int)((n - t0) < TK ? (n - t0) : TK);
        for (int tt = 0; tt < tc; ++tt) {
            const AT lj = (AT)Lt[tt * 64 + j];
#pragma unroll
            for (int q = 0; q < 16; ++q) g[q] += (AT)Lt[tt * 64 + i0 + 4 * q] * lj;
        }
    }
    // ---- G + lambda I on the real indices, identity on the padding
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int i = i0 + 4 * q;
        if (i < kc_real && j < kc_real) g[q] += (i == j) ? (AT)lambda : AT(0);
        else g[q] = (i == j) ? AT(1) : AT(0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q)
        if (i0 + 4 * q == j) vec[0][j] = g[q];  // the diagonal, one owner per entry
    __syncthreads();
    if (tid == 0) {
        AT dmax = AT(0);
        for (int i = 0; i < kc; ++i) dmax = dmax > vec[0][i] ? dmax : vec[0][i];
        thresh = lambda > 0.f ? AT(0) : (AT)kc * AT(2.3e-16) * dmax;
        if (!(dmax > AT(0))) fail = 1;
    }
    __syncthreads();
    const AT th = thresh;
    // ---- Cholesky G = C C^T (lower), right-looking, one barrier per column
    for (int k = 0; k < kc; ++k) {
        AT *colk = vec[k & 1];
        if (j == k) {
#pragma unroll
            for (int q = 0; q < 16; ++q) colk[i0 + 4 * q] = g[q];
        }
        __syncthreads();
        AT pk = colk[k];
        if (k < kc_real && !(pk > th)) {
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
#pragma unroll
    for (int q = 0; q < 16; ++q) g[q] = (j > i0 + 4 * q) ? AT(0) : g[q];
    __syncthreads();
    // ---- C^-1 by in-place Gauss-Jordan (stays lower-triangular)
    for (int k = 0; k < kc; ++k) {
        AT *colk = vec[k & 1];
        AT *rowk = rowv[k & 1];
        if (j == k) {
#pragma unroll
            for (int q = 0; q < 16; ++q) colk[i0 + 4 * q] = g[q];
        }
        if ((k & 3) == i0) {
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
    const bool failed = fail != 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) G[(i0 + 4 * q) * GS + j] = failed ? AT(0) : g[q];
    __syncthreads();
    // ---- one token per thread: q_t = C^-1 l_t
    float *Qb = Qt + b * kc * npad;
    for (int64_t t = tid; t < npad; t += NT) {
        AT l[64];
#pragma unroll
        for (int c = 0; c < 64; ++c) l[c] = (t < n && c < kc) ? (AT)Lb[t * ldt + c] : AT(0);
        for (int i = 0; i < kc; ++i) {
            AT sum = AT(0);
#pragma unroll
            for (int c = 0; c < 64; ++c) sum += G[i * GS + c] * l[c];
            Qb[(int64_t)i * npad + t] = (float)sum;
            if (t < n) Lb[t * ldt + i] = (float)sum;
        }
    }
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

template <>
hipError_t launch_gram_q<bf16>(bf16 *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real,
                               int kc, float lambda, bf16 *Qt, int *flags, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    const dim3 grid((unsigned)((npad + NT - 1) / NT), (unsigned)B);
    switch (kc) {
    case 16: hipLaunchKernelGGL(cholq_kernel<16>, grid, dim3(NT), 0, st, T, ldt, off, n, npad, kc_real, lambda, Qt, flags); break;
    case 32: hipLaunchKernelGGL(cholq_kernel<32>, grid, dim3(NT), 0, st, T, ldt, off, n, npad, kc_real, lambda, Qt, flags); break;
    case 48: hipLaunchKernelGGL(cholq_kernel<48>, grid, dim3(NT), 0, st, T, ldt, off, n, npad, kc_real, lambda, Qt, flags); break;
    case 64: hipLaunchKernelGGL(cholq_kernel<64>, grid, dim3(NT), 0, st, T, ldt, off, n, npad, kc_real, lambda, Qt, flags); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <>
hipError_t launch_gram_q<float>(float *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real,
                                int kc, float lambda, float *Qt, int *flags, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    if (kc < 1 || kc > 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gram_q_f32_kernel, dim3((unsigned)B), dim3(NT), 0, st, T, ldt, off, n, npad, kc_real, kc,
                       lambda, Qt, flags);
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

template hipError_t launch_mprime<bf16>(const bf16 *, const bf16 *, int64_t, int64_t, int64_t, int64_t, int, bf16 *,
                                        hipStream_t);
template hipError_t launch_mprime<float>(const float *, const float *, int64_t, int64_t, int64_t, int64_t, int,
                                         float *, hipStream_t);

}  // namespace dyra
