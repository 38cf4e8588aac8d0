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
//            all n tokens of b (the block's own tokens are loaded once, into
//            registers, and serve both G and the elimination), then every
//            wavefront factors G with one matrix row per lane and, in the same
//            elimination steps, turns its 64 token rows of L1_b into rows of
//            Q_b: factoring [G; L1_b] leaves L1_b C^-T in the lower block.  The
//            pivot row's entries reach all lanes through v_readlane, so the
//            factorisation has no barrier and no LDS traffic.
//   gram_q (float32)  one workgroup per instance, all in float64: G, a
//            right-looking Cholesky and the inverse C^-1 with 16 matrix entries
//            per thread, then q_t = C^-1 l_t per token, written both in place
//            and transposed (Qt) for the float32 mprime.
//   mprime (bf16)  workgroup (instance b, 256 input features):
//            M'_b = Q_b^T X_b with X_b and Q_b staged row-major through LDS.
//   mprime (float32)  the same product from Q_b^T stored token-contiguous.
#include "dyra_kernels.h"

#include "elim.h"
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
        // unconditional load of a clamped entry, zeroed after (a guarded load
        // compiles to a branch and a full wait)
        const bool ok = t0 + tok < tokens && col0 + j0 < cols_valid;
        v.u = *reinterpret_cast<const uint4 *>(src + (t0 + tok < tokens ? t0 + tok : tokens - 1) * ld +
                                               (col0 + j0 < cols_valid ? col0 + j0 : 0));
        if (!ok) v.u = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < VEC; ++q) dst[(j0 + q) * ST + tok] = v.e[q];
    }
}

// ---------------------------------------------------------------- bf16 path
template <int KC>
__global__ __launch_bounds__(NT) void cholq_kernel(bf16 *__restrict__ T, int64_t ldt, int64_t off, int64_t n,
                                                   int kc_real, float lambda, int *__restrict__ flags,
                                                   double *__restrict__ Cout) {
    constexpr int GS = 68;        // row stride (floats) of G in LDS
    constexpr int TT = NT;        // tokens per Gram chunk = tokens per workgroup
    constexpr int ST = TT + 8;    // row stride (bf16) of the transposed chunk [feature][token]
    constexpr int NBLK = (KC + 31) / 32;
    constexpr int NV = KC / 8;    // 16-byte vectors per token row
    __shared__ __align__(16) bf16 Lt[64 * ST];
    __shared__ __align__(16) float Gs[64 * GS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int64_t b = blockIdx.y;
    bf16 *const Tb = T + b * n * ldt + off;  // token t of instance b: Tb + t * ldt
    DYRA_PHASE_MARK(0);

    // this thread's token row of L1_b, requested first so that its latency
    // overlaps the set-up (tokens past n read as zero)
    const int64_t tbase = (int64_t)blockIdx.x * TT;
    const int64_t t = tbase + tid;
    const bool tin = t < n;
    uint4 lraw[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const uint4 x = *reinterpret_cast<const uint4 *>(Tb + (tin ? t * ldt : 0) + 8 * v);
        lraw[v] = tin ? x : make_uint4(0, 0, 0, 0);
    }
    // features KC .. 32 NBLK - 1 of the transposed chunk are MFMA padding
    if (KC % 32 != 0) {
        for (int e = tid; e < (32 * NBLK - KC) * ST; e += NT) Lt[KC * ST + e] = bf16(0.f);
    }

    // ---- G = L1_b^T L1_b over all n tokens, 32x32 blocks on MFMA; the
    // workgroup's own chunk comes from lraw, others (n > TT) are loaded
    const int wm = wave >> 1, wn = wave & 1;
    const bool gact = wm < NBLK && wn < NBLK;
    f32x16 acc = f32x16{};
    const int64_t nch = (n + TT - 1) / TT;
    for (int64_t ch = 0; ch < nch; ++ch) {
        const int64_t c0 = ch * TT;
        uint4 v[NV];
        if (c0 == tbase) {
#pragma unroll
            for (int q = 0; q < NV; ++q) v[q] = lraw[q];
        } else {
            const bool ok = c0 + tid < n;
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const uint4 x = *reinterpret_cast<const uint4 *>(Tb + (ok ? (c0 + tid) * ldt : 0) + 8 * q);
                v[q] = ok ? x : make_uint4(0, 0, 0, 0);
            }
        }
        __syncthreads();  // the previous chunk's MFMA reads are done
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            union { uint4 u; bf16 e[8]; } w;
            w.u = v[q];
#pragma unroll
            for (int e = 0; e < 8; ++e) Lt[(8 * q + e) * ST + tid] = w.e[e];
        }
        __syncthreads();
        if (gact) {
#pragma unroll 4
            for (int kk = 0; kk < TT; kk += 16)
                acc = mma16(acc, ld_frag(Lt + (wm * 32 + lr) * ST + kk + lk), ld_frag(Lt + (wn * 32 + lr) * ST + kk + lk));
        }
    }
    if (gact) {
#pragma unroll
        for (int q = 0; q < 16; ++q) Gs[(wm * 32 + acc_row(lane, q)) * GS + wn * 32 + lr] = acc[q];
    }
    __syncthreads();
    DYRA_PHASE_MARK(1);

    // ---- lane i holds row i of G + lambda I (identity rows past kc_real)
    const int i = lane;
    float g[KC];
#pragma unroll
    for (int m = 0; m < KC; m += 4) {
        const float4 x = *reinterpret_cast<const float4 *>(&Gs[(i < KC ? i : 0) * GS + m]);
        g[m] = x.x; g[m + 1] = x.y; g[m + 2] = x.z; g[m + 3] = x.w;
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
    float l[KC];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        union { uint4 u; bf16 e[8]; } w;
        w.u = lraw[q];
#pragma unroll
        for (int e = 0; e < 8; ++e) l[8 * q + e] = (float)w.e[e];
    }
    DYRA_PHASE_MARK(2);

    // ---- elimination: step k takes pivot row k (lane k) to all lanes
    elim_step<KC, 0>(g, l, kc_real, th, fail);
    DYRA_PHASE_MARK(3);

    // ---- Q_b rows in place of L1_b
    if (tin) {
#pragma unroll
        for (int m = 0; m < KC; m += 8) {
            union { uint4 u; bf16 e[8]; } w;
#pragma unroll
            for (int q = 0; q < 8; ++q) w.e[q] = fail ? bf16(0.f) : (bf16)l[m + q];
            *reinterpret_cast<uint4 *>(Tb + t * ldt + m) = w.u;
        }
    }
    if (blockIdx.x == 0 && tid == 0) flags[b] = fail ? 1 : 0;
    // the Cholesky factor itself (lane i holds row i of C in g[0..i]) for the
    // L updates of further ALS steps
    if (Cout && blockIdx.x == 0 && wave == 0 && i < KC) {
        double *Cr = Cout + ((int64_t)b * KC + i) * KC;
#pragma unroll
        for (int m = 0; m < KC; ++m) Cr[m] = m <= i ? (double)g[m] : 0.0;
    }
    DYRA_PHASE_MARK(4);
}

// ------------------------------------------------------------- float32 path
__global__ __launch_bounds__(NT) void gram_q_f32_kernel(float *__restrict__ T, int64_t ldt, int64_t off, int64_t n,
                                                        int64_t npad, int kc_real, int kc, float lambda,
                                                        float *__restrict__ Qt, int *__restrict__ flags,
                                                        double *__restrict__ Cout) {
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
        // loads are unconditional (clamped to a valid entry, zeroed after):
        // a guarded load compiles to a branch and a full wait per element
        for (int e = tid; e < TK * 64; e += NT) {
            const int tt = e >> 6, c = e & 63;
            const bool ok = t0 + tt < n && c < kc;
            const float v = Lb[(t0 + tt < n ? t0 + tt : n - 1) * ldt + (c < kc ? c : 0)];
            Lt[tt * 64 + c] = ok ? v : 0.f;
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
    if (Cout) {
#pragma unroll
        for (int q = 0; q < 16; ++q)
            if (i0 + 4 * q < kc && j < kc) Cout[((int64_t)b * kc + i0 + 4 * q) * kc + j] = g[q];
    }
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
        const int64_t tc = t < n ? t : n - 1;
#pragma unroll
        for (int c = 0; c < 64; ++c) {
            const float v = Lb[tc * ldt + (c < kc ? c : 0)];
            l[c] = (t < n && c < kc) ? (AT)v : AT(0);
        }
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

// ------------------------------------------------- M'_b = Q_b^T X_b, bf16
// Workgroup (256 input features, instance b); token slices of 32 rows of X_b
// and of Q_b are loaded into registers two slices ahead, written to a double
// buffered LDS stage row-major (as stored), and the token-contiguous MFMA
// fragments come out of LDS through transposing reads (ds_read_b64_tr_b16: in
// each group of 16 lanes, lane i receives element i % 4 of the 8-byte rows
// addressed by lanes i / 4 + 4 q, q = 0..3, so 16 lanes addressing a 4-token x
// 16-feature block receive one feature each, four tokens deep).  LDS chunk
// swizzles keep those reads on distinct banks: X rows (512 bytes) hold chunk c
// at c ^ 4 (r % 4), Q rows (128 bytes) at c ^ 4 ((r / 2) % 2).  The finished
// 64 x 256 block of M'_b goes back through LDS so that it leaves as whole
// 512-byte row segments.
//
// Register staging keeps more bytes in flight per compute unit than the
// direct-to-LDS loads of the GEMMs: this kernel streams X_b once from HBM
// and is bound by that read, not by the MFMA work.
typedef short v4i16 __attribute__((ext_vector_type(4)));
constexpr int kMprimeFeatures = 256;  // features per mprime workgroup (128 measured no faster)

__device__ __forceinline__ uint2 lds_tr16(const char *p) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(__attribute__((address_space(3))) char *)p);
    union { v4i16 s; uint2 u; } w;
    w.s = v;
    return w.u;
}

template <int KC, int CW>
__global__ __launch_bounds__(NT) void mprime_tr_kernel(const bf16 *__restrict__ X, const bf16 *__restrict__ T,
                                                       int64_t ldt, int64_t off, int64_t n, int64_t c1,
                                                       bf16 *__restrict__ Mp) {
    // CW features per workgroup, CW / 4 per wavefront
    constexpr int TS = 32;                  // tokens per slice
    constexpr int RB = CW * 2;              // bytes per X row in LDS
    constexpr int XBYTES = TS * RB;         // 16 KB
    constexpr int QROW = 128;               // bytes per Q row in LDS (64 columns)
    constexpr int STAGE = XBYTES + TS * QROW;
    constexpr int LX = XBYTES / 16 / NT;    // 16-byte X loads per thread and slice (4)
    constexpr int CPX = RB / 16;            // 16-byte chunks per X row
    constexpr int NKB = (KC + 31) / 32;     // 32-row blocks of M'_b
    constexpr int MS = CW + 8;              // row stride (elements) of the staged M'_b block
    constexpr int JB = CW / 128;            // 32-feature blocks per wavefront
    static_assert(CW == 128 || CW == 256, "feature block");
    static_assert(TS * QROW == 16 * NT && KC * MS * 2 <= 2 * STAGE, "layout");
    __shared__ __align__(16) char smem[2 * STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t b = blockIdx.y;
    const int64_t f0 = (int64_t)blockIdx.x * CW;
    const bf16 *Xb = X + b * n * c1;
    const bf16 *Qb = T + b * n * ldt + off;
    const int64_t S = (n + TS - 1) / TS;

    // thread tid loads X chunks q * 256 + tid (row-major over the slice) and
    // Q chunk tid; rows past n repeat row n - 1 (masked in the product),
    // features past c1 read feature 0 (never stored).  Two register sets hold
    // the next two slices, so two slices' loads are in flight during a
    // slice's MFMAs; the slice loop is unrolled by two so that every index
    // into the sets is a constant.
    u32x4 reg[2][LX + 1];
    auto load = [&](int64_t s, u32x4 (&rg)[LX + 1]) __attribute__((always_inline)) {
        const int64_t t0 = s * TS;
#pragma unroll
        for (int q = 0; q < LX; ++q) {
            const int e = q * NT + tid, row = e / CPX, c = e % CPX;
            const int64_t t = t0 + row < n ? t0 + row : n - 1;
            const int64_t f = f0 + 8 * c < c1 ? f0 + 8 * c : 0;
            rg[q] = *reinterpret_cast<const u32x4 *>(Xb + t * c1 + f);
        }
        const int row = tid >> 3, c = tid & 7;
        const int64_t t = t0 + row < n ? t0 + row : n - 1;
        rg[LX] = *reinterpret_cast<const u32x4 *>(Qb + t * ldt + (8 * c < KC ? 8 * c : 0));
    };
    auto stage = [&](int slot, const u32x4 (&rg)[LX + 1]) __attribute__((always_inline)) {
        char *dst = smem + slot * STAGE;
#pragma unroll
        for (int q = 0; q < LX; ++q) {
            const int e = q * NT + tid, row = e / CPX, c = e % CPX;
            *reinterpret_cast<u32x4 *>(dst + row * RB + ((c ^ (4 * (row & 3))) << 4)) = rg[q];
        }
        const int row = tid >> 3, c = tid & 7;
        *reinterpret_cast<u32x4 *>(dst + XBYTES + row * QROW + ((c ^ (4 * ((row >> 1) & 1))) << 4)) = rg[LX];
    };

    // per-lane transposing-read offsets: 16-lane group g = lane / 16 covers
    // tokens 8 (g / 2) + 4 u + (lane % 16) / 4 and columns 16 (g % 2) + 4 (lane % 4) + 0..3
    const int g = lane >> 4, rq = (lane & 15) >> 2, cq = 4 * (lane & 3);
    const int hcol = 16 * (g & 1) + cq;  // column inside a 32-column block
    auto xoff = [&](int row, int col) { return row * RB + (((col >> 3) ^ (4 * (row & 3))) << 4) + (col & 7) * 2; };
    auto qoff = [&](int row, int col) { return row * QROW + (((col >> 3) ^ (4 * ((row >> 1) & 1))) << 4) + (col & 7) * 2; };

    f32x16 acc[JB][NKB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int ib = 0; ib < NKB; ++ib) acc[jb][ib] = f32x16{};

    // slice s (register set and LDS stage s % 2): stage it (waits for its
    // loads), barrier, request slice s + 2 into the set just staged, multiply.
    // The LDS stage written at slice s + 2 was last read at slice s, before
    // the barrier of slice s + 1.  The request is unconditional (past the last
    // slice it rereads row n - 1): with the same loads outstanding on every
    // path, the wait before staging a set covers that set's loads only.
    auto slice = [&](int64_t s, int slot, u32x4 (&rg)[LX + 1]) __attribute__((always_inline)) {
        stage(slot, rg);
        __syncthreads();
        load(s + 2, rg);
        const char *sx = smem + slot * STAGE;
        const char *sq = sx + XBYTES;
        const int64_t t0 = s * TS;
        const bool tail = t0 + TS > n;
#pragma unroll
        for (int h = 0; h < TS / 16; ++h) {
            bf16x8 fx[JB], fq[NKB];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int row = 16 * h + 8 * (g >> 1) + 4 * u + rq;
#pragma unroll
                for (int jb = 0; jb < JB; ++jb)
                    reinterpret_cast<uint2 *>(&fx[jb])[u] = lds_tr16(sx + xoff(row, 32 * JB * wave + 32 * jb + hcol));
#pragma unroll
                for (int ib = 0; ib < NKB; ++ib)
                    reinterpret_cast<uint2 *>(&fq[ib])[u] = lds_tr16(sq + qoff(row, 32 * ib + hcol));
            }
            // Q columns past KC and tokens past n contribute nothing
#pragma unroll
            for (int ib = 0; ib < NKB; ++ib) {
                if (KC % 32 != 0 && 32 * ib + (lane & 31) >= KC) fq[ib] = bf16x8{};
                if (tail) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (t0 + 16 * h + 8 * (lane >> 5) + e >= n) fq[ib][e] = bf16(0.f);
                }
            }
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                for (int ib = 0; ib < NKB; ++ib) acc[jb][ib] = mma16(acc[jb][ib], fx[jb], fq[ib]);
        }
    };
    load(0, reg[0]);
    __builtin_amdgcn_sched_barrier(0);  // set 0's loads stay older than set 1's, as in the loop
    load(1, reg[1]);
    // pairs of slices, then an odd last one (the loop body itself has no
    // branch around a half, which would merge load orders at its head)
    int64_t s = 0;
    for (; s + 1 < S; s += 2) {
        slice(s, 0, reg[0]);
        slice(s + 1, 1, reg[1]);
    }
    if (s < S) slice(s, 0, reg[0]);

    // lane holds row kk = 32 ib + lane % 32 of M'_b and, per register group q,
    // four consecutive features; staged as [kk][feature], stored by rows
    __syncthreads();
    bf16 *ms = reinterpret_cast<bf16 *>(smem);
#pragma unroll
    for (int ib = 0; ib < NKB; ++ib) {
        const int kk = 32 * ib + (lane & 31);
        if (kk >= KC) continue;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                union { uint2 u; bf16 e[4]; } w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w.e[e] = (bf16)acc[jb][ib][4 * q + e];
                *reinterpret_cast<uint2 *>(ms + kk * MS + 32 * JB * wave + 32 * jb + acc_row(lane, 4 * q)) = w.u;
            }
    }
    __syncthreads();
    constexpr int CPM = CW / 8;  // 16-byte chunks per M'_b row segment
#pragma unroll
    for (int q = 0; q < KC * CPM / NT; ++q) {
        const int e = q * NT + tid, row = e / CPM, c = e % CPM;
        if (f0 + 8 * c < c1)
            *reinterpret_cast<u32x4 *>(Mp + (b * KC + row) * c1 + f0 + 8 * c) =
                *reinterpret_cast<const u32x4 *>(ms + row * MS + 8 * c);
    }
}

}  // namespace

template <>
hipError_t launch_gram_q<bf16>(bf16 *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real,
                               int kc, float lambda, bf16 *, int *flags, double *Cout, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    const dim3 grid((unsigned)((npad + NT - 1) / NT), (unsigned)B);
    switch (kc) {
    case 16: hipLaunchKernelGGL(cholq_kernel<16>, grid, dim3(NT), 0, st, T, ldt, off, n, kc_real, lambda, flags, Cout); break;
    case 32: hipLaunchKernelGGL(cholq_kernel<32>, grid, dim3(NT), 0, st, T, ldt, off, n, kc_real, lambda, flags, Cout); break;
    case 48: hipLaunchKernelGGL(cholq_kernel<48>, grid, dim3(NT), 0, st, T, ldt, off, n, kc_real, lambda, flags, Cout); break;
    case 64: hipLaunchKernelGGL(cholq_kernel<64>, grid, dim3(NT), 0, st, T, ldt, off, n, kc_real, lambda, flags, Cout); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <>
hipError_t launch_gram_q<float>(float *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real,
                                int kc, float lambda, float *Qt, int *flags, double *Cout, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    if (kc < 1 || kc > 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gram_q_f32_kernel, dim3((unsigned)B), dim3(NT), 0, st, T, ldt, off, n, npad, kc_real, kc,
                       lambda, Qt, flags, Cout);
    return hipGetLastError();
}

template <>
hipError_t launch_mprime<bf16>(const bf16 *X, const bf16 *T, int64_t ldt, int64_t off, const bf16 *, int64_t B,
                               int64_t n, int64_t, int64_t c1, int kc, bf16 *Mp, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    constexpr int CW = kMprimeFeatures;
    const dim3 grid((unsigned)((c1 + CW - 1) / CW), (unsigned)B);
    switch (kc) {
    case 16: hipLaunchKernelGGL((mprime_tr_kernel<16, CW>), grid, dim3(NT), 0, st, X, T, ldt, off, n, c1, Mp); break;
    case 32: hipLaunchKernelGGL((mprime_tr_kernel<32, CW>), grid, dim3(NT), 0, st, X, T, ldt, off, n, c1, Mp); break;
    case 48: hipLaunchKernelGGL((mprime_tr_kernel<48, CW>), grid, dim3(NT), 0, st, X, T, ldt, off, n, c1, Mp); break;
    case 64: hipLaunchKernelGGL((mprime_tr_kernel<64, CW>), grid, dim3(NT), 0, st, X, T, ldt, off, n, c1, Mp); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <>
hipError_t launch_mprime<float>(const float *X, const float *, int64_t, int64_t, const float *Qt, int64_t B,
                                int64_t n, int64_t npad, int64_t c1, int kc, float *Mp, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL((mprime_kernel<float>), dim3((unsigned)((c1 + 255) / 256), (unsigned)B), dim3(NT), 0, st, X,
                       Qt, n, npad, c1, kc, Mp);
    return hipGetLastError();
}

}  // namespace dyra
