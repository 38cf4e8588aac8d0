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
//   gram_chol (bf16)  workgroup per instance b: G by MFMA over all n tokens
//            of b, then its Cholesky factor C in one wavefront with one matrix
//            row per lane (the pivot row reaches all lanes through
//            v_readlane: no barrier, no LDS traffic), stored column by column.
//   q_apply (bf16)  workgroup per (64 tokens, instance b): Q_b = L1_b C^-T in
//            place by forward substitution, each token row over a quad of
//            lanes, C staged in LDS.  G is complete before any row of T is
//            rewritten: the two are separate launches.
//   gram_q (float32)  one workgroup per instance, all in float64: G, a
//            right-looking Cholesky and the inverse C^-1 with 16 matrix entries
//            per thread, then q_t = C^-1 l_t per token, written both in place
//            and transposed (Qt) for the float32 mprime.
//   mprime (bf16)  workgroup (instance b, 256 input features):
//            M'_b = Q_b^T X_b with X_b and Q_b staged row-major through LDS.
//   mprime (float32)  the same product from Q_b^T stored token-contiguous.
#include "dyra_kernels.h"

#include "elim.h"
#include "lanes.h"
#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;
constexpr int TK = 32;  // tokens per slice of the token contraction (mprime)

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
// Lane-per-row Cholesky step K of a matrix held one row per lane (g of lane
// i = row i): the pivot row's entries reach every lane through v_readlane in
// batches of 8.  After all steps g[0..i] of lane i is row i of the lower
// factor C (G = C C^T); entries past the diagonal are left over.
template <int KC, int K, int M0>
__device__ __forceinline__ void chol_batch(float (&g)[KC], float a) {
    constexpr int CNT = (KC - M0) < 8 ? (KC - M0) : 8;
    float sv[CNT];
#pragma unroll
    for (int u = 0; u < CNT; ++u) sv[u] = bcast(g[M0 + u], K);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CNT; ++u) g[M0 + u] = fmaf(-a, sv[u], g[M0 + u]);
#pragma unroll
    for (int u = 0; u < CNT; ++u) asm volatile("" : "+v"(g[M0 + u]));
    if constexpr (M0 + 8 < KC) chol_batch<KC, K, M0 + 8>(g, a);
}

template <int KC, int K>
__device__ __forceinline__ void chol_step(float (&g)[KC], int kc_real, float th, bool &fail) {
    if constexpr (K < KC) {
        float pk = bcast(g[K], K);
        const bool bad = K < kc_real && !(pk > th);  // padding pivots are 1
        fail = fail || bad;
        pk = bad ? 1.f : pk;
        const float a = g[K] * __builtin_amdgcn_rcpf(pk);  // G[i][K] / G[K][K]
        g[K] = g[K] * __builtin_amdgcn_rsqf(pk);           // C[i][K]
        if constexpr (K + 1 < KC) chol_batch<KC, K, K + 1>(g, a);
        chol_step<KC, K + 1>(g, kc_real, th, fail);
    }
}

// Sizes of gram_chol_kernel for a padded correction rank KC (a multiple of 16,
// at most 256): G is factored as a KP x KP matrix (KC rounded up to whole
// 32-wide panels, identity on the padding), held in LDS up to KP = 128 and in
// the workspace (L2) above; token chunks of TT rows are staged per pass.
template <int KC> constexpr int gram_kp() { return (KC + 31) / 32 * 32; }
template <int KC> constexpr bool gram_g_in_lds() { return gram_kp<KC>() <= 128; }
template <int KC> constexpr int gram_tokens() { return gram_kp<KC>() <= 64 ? 256 : (gram_kp<KC>() <= 128 ? 128 : 64); }

// Per instance b (one workgroup of four wavefronts):
//  1. G = L1_b^T L1_b + lambda I over all n tokens: token chunks are loaded,
//     written transposed to LDS ([feature][token]) and multiplied on MFMA, the
//     lower 32 x 32 blocks of G dealt round-robin to the wavefronts; the next
//     chunk's loads are in flight during the current chunk's MFMAs.
//  2. Its Cholesky factor C by 32-wide panels (right-looking, blocked): each
//     wavefront eliminates [G_pp; 64 rows of G below the panel] with one row
//     per lane (elim_step: the pivot rows reach every lane through
//     v_readlane, each wavefront factoring the 32 x 32 diagonal block for
//     itself), which leaves the panel's rows of C; the trailing matrix then
//     loses C_below C_below^T, formed on float32 MFMA from the panel staged in
//     LDS.
// C is stored column by column, Ct[b][m][i] = C[i][m] (i > m), Ct[b][m][m] =
// 1 / C[m][m], zero above: the order q_apply_kernel reads it in (not with FUSE,
// which needs no second launch).  The kernel
// only reads T; Q is formed by a later launch, so no workgroup sees rows
// another one rewrites.
// GONLY: stop after G, written whole (both triangles) to Gw for the
// Newton-Schulz solve.
// FUSE (n <= 256, KC <= 64): no other workgroup reads the instance's rows,
// so the workgroup also forms Q = L1 C^-T and writes it over L1: one launch
// instead of two.  C^-1 comes out of the elimination itself: wavefront 0's
// lanes 32..63, idle as pivot rows, carry identity rows through each 32-wide
// panel and leave the rows of the diagonal block's C_pp^-T; with two panels
// the block below the diagonal of C^-1 is -C_11^-1 C_10 C_00^-1.  Then
// Q^T = C^-1 L1^T on MFMA, C^-1 split into two bf16 terms (high part and
// rounding remainder) against the exact bf16 L1 rows, each wavefront taking
// 64 tokens.
template <int KC, bool GONLY = false, bool FUSE = false>
__global__ __launch_bounds__(NT) void gram_chol_kernel(const bf16 *T, int64_t ldt, int64_t off,
                                                       int64_t n, int kc_real, float lambda, float *__restrict__ Ct,
                                                       float *__restrict__ Gw, int *__restrict__ flags,
                                                       double *__restrict__ Cout) {
    static_assert(KC % 16 == 0 && KC >= 16 && KC <= 256, "correction rank");
    constexpr int KP = gram_kp<KC>();
    constexpr int NBB = KP / 32;                  // 32-blocks per side
    constexpr int NLOW = NBB * (NBB + 1) / 2;     // lower blocks of G
    constexpr int NQ = (NLOW + 3) / 4;            // G blocks per wavefront
    constexpr int TT = gram_tokens<KC>();         // tokens per chunk
    constexpr int ST = TT + 8;                    // row stride (bf16) of the transposed chunk
    constexpr int VPR = KC / 8;                   // 16-byte vectors per token row
    constexpr int TOT = TT * VPR;                 // vectors per chunk
    constexpr int NL = (TOT + NT - 1) / NT;       // vectors per thread
    constexpr bool GLDS = !GONLY && gram_g_in_lds<KC>();
    constexpr int GS = GLDS ? KP + 4 : KP;        // row stride (floats) of G
    constexpr int CBS = 36;                       // row stride (floats) of the staged panel
    __shared__ __align__(16) bf16 Lt[KP * ST];
    __shared__ __align__(16) float Gsh[GLDS ? KP * GS : 4];
    __shared__ __align__(16) float Cb[(KP > 32 ? KP - 32 : 1) * CBS];
    // FUSE: C row-major (Cs[i][m] = C[i][m] below the diagonal, 1 / C[i][i] on
    // it) for the in-kernel substitution
    static_assert(!FUSE || (KP <= 64 && TT >= NT && !GONLY), "fused Q: one token chunk, 64 tokens per wavefront");
    constexpr int CSS = KP + 4;
    __shared__ __align__(16) float Cs[FUSE ? KP * CSS : 4];
    // FUSE: C^-1 row-major (Ci[j][m]; its upper-right 32 x 32 block is never
    // written nor read) and, with two panels, C_10 C_00^-1
    __shared__ __align__(16) float Ci[FUSE ? KP * CSS : 4];
    __shared__ float Pm[FUSE && KP == 64 ? 32 * 33 : 1];
    __shared__ float sh_dmax;
    __shared__ int sh_fail;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int64_t b = blockIdx.x;
    const bf16 *const Tb = T + b * n * ldt + off;  // token t of instance b: Tb + t * ldt
    float *const G = GLDS ? Gsh : Gw + b * KP * KP;
    auto blk = [](int q, int &bi, int &bj) {  // q-th lower block, row by row
        bi = 0;
        while ((bi + 1) * (bi + 2) / 2 <= q) ++bi;
        bj = q - bi * (bi + 1) / 2;
    };

    // features KC .. KP - 1 of the transposed chunk are MFMA padding
    if (KC != KP) {
        for (int e = tid; e < (KP - KC) * ST; e += NT) Lt[KC * ST + e] = bf16(0.f);
    }
    // a chunk's token rows, requested unconditionally (rows past n reread
    // row n - 1 and are zeroed when staged)
    auto load = [&](int64_t c0, u32x4 (&v)[NL]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const int e = q * NT + tid < TOT ? q * NT + tid : 0;
            const int tok = e % TT, vec = e / TT;
            const int64_t t = c0 + tok < n ? c0 + tok : n - 1;
            v[q] = *reinterpret_cast<const u32x4 *>(Tb + t * ldt + 8 * vec);
        }
    };
    f32x16 acc[NQ];
#pragma unroll
    for (int s = 0; s < NQ; ++s) acc[s] = f32x16{};
    const int64_t nch = (n + TT - 1) / TT;
    u32x4 v[NL];
    load(0, v);
    for (int64_t ch = 0; ch < nch; ++ch) {
        __syncthreads();  // the previous chunk's MFMA reads are done
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const int e = q * NT + tid;
            if (TOT % NT == 0 || e < TOT) {
                const int tok = e % TT, vec = e / TT;
                const bool in = ch * TT + tok < n;
                union { u32x4 u; bf16 h[8]; } w;
                w.u = v[q];
#pragma unroll
                for (int j = 0; j < 8; ++j) Lt[(8 * vec + j) * ST + tok] = in ? w.h[j] : bf16(0.f);
            }
        }
        __syncthreads();
        if (ch + 1 < nch) load((ch + 1) * TT, v);
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            const int q = wave + 4 * s;
            if (q < NLOW) {
                int bi, bj;
                blk(q, bi, bj);
                const bf16 *pa = Lt + (bi * 32 + lr) * ST + lk, *pb = Lt + (bj * 32 + lr) * ST + lk;
#pragma unroll 4
                for (int kk = 0; kk < TT; kk += 16) acc[s] = mma16(acc[s], ld_frag(pa + kk), ld_frag(pb + kk));
            }
        }
    }
    // G + lambda I on the real indices, identity on the padding (lower blocks)
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
        const int q = wave + 4 * s;
        if (q < NLOW) {
            int bi, bj;
            blk(q, bi, bj);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int i = bi * 32 + acc_row(lane, t), j = bj * 32 + lr;
                const bool real = i < kc_real && j < kc_real;
                const float gv = real ? acc[s][t] + (i == j ? lambda : 0.f) : (i == j ? 1.f : 0.f);
                G[i * GS + j] = gv;
                if (GONLY && bi != bj) G[j * GS + i] = gv;
            }
        }
    }
    if constexpr (GONLY) return;
    if (Cout) {  // its upper part stays zero; the panels fill the rest
        for (int e = tid; e < KC * KC; e += NT) Cout[b * KC * KC + e] = 0.0;
    }
    __syncthreads();
    // a pivot at or below the working precision times the largest diagonal
    // marks a numerically singular G (possible only for lambda = 0)
    if (wave == 0) {
        float d = 0.f;
        for (int i = lane; i < kc_real; i += 64) d = fmaxf(d, G[i * GS + i]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) d = fmaxf(d, __shfl_xor(d, o));
        if (lane == 0) sh_dmax = d;
    }
    __syncthreads();
    const float dmax = sh_dmax;
    const float th = lambda > 0.f ? 0.f : (float)KC * 1.2e-7f * dmax;
    bool fail = !(dmax > 0.f);
    float *const Cb_ = Ct + b * KC * KC;

    for (int p0 = 0; p0 < KP; p0 += 32) {
        const int below = KP - p0 - 32;             // rows under the panel
        const bool has_l = 64 * wave < below;
        if (wave == 0 || has_l) {
            float g[32], l[32];
            const int rg = p0 + (lane < 32 ? lane : 0);
            const int rl = p0 + 32 + 64 * wave + lane;
            const bool lin = rl < KP;
            // FUSE: wavefront 0's lanes 32..63 hold identity rows (data rows
            // that the elimination turns into rows of C_pp^-T)
            const bool idrow = FUSE && wave == 0 && lane >= 32;
#pragma unroll
            for (int m = 0; m < 32; m += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&G[rg * GS + p0 + m]);
                const f32x4 y = *reinterpret_cast<const f32x4 *>(&G[(lin ? rl : rg) * GS + p0 + m]);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    g[m + u] = lane < 32 ? x[u] : (idrow && m + u == lane - 32 ? 1.f : 0.f);
                    l[m + u] = lin ? y[u] : 0.f;
                }
            }
            bool f = false;
            if (has_l) elim_step<32, 0>(g, l, kc_real - p0, th, f);
            else chol_step<32, 0>(g, kc_real - p0, th, f);
            if (wave == 0) fail = fail || f;
            // the panel's rows of C: the diagonal block (wavefront 0) and the
            // rows below it (every wavefront), by columns into Ct
            if (wave == 0 && lane < 32 && p0 + lane < KC) {
                const int i = p0 + lane;
#pragma unroll
                for (int m = 0; m < 32; ++m) {
                    if (p0 + m < KC) {
                        const float c = m < lane ? g[m] : (m == lane ? __builtin_amdgcn_rcpf(g[m]) : 0.f);
                        if constexpr (!FUSE) Cb_[(p0 + m) * KC + i] = c;  // for q_apply_kernel
                        if constexpr (FUSE) Cs[i * CSS + p0 + m] = c;
                        if (Cout && m <= lane) Cout[(b * KC + i) * KC + p0 + m] = (double)g[m];
                    }
                }
            }
            if (idrow) {
                // lane 32 + i holds row i of C_pp^-T: column i of C_pp^-1
                const int i = lane - 32;
#pragma unroll
                for (int m = 0; m < 32; ++m) Ci[(p0 + m) * CSS + p0 + i] = g[m];
            }
            if (has_l && lin) {
                if (rl < KC) {
#pragma unroll
                    for (int m = 0; m < 32; ++m) {
                        if (p0 + m < KC) {
                            if constexpr (!FUSE) Cb_[(p0 + m) * KC + rl] = l[m];
                            if constexpr (FUSE) Cs[rl * CSS + p0 + m] = l[m];
                            if (Cout) Cout[(b * KC + rl) * KC + p0 + m] = (double)l[m];
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < 32; m += 4)
                    *reinterpret_cast<f32x4 *>(&Cb[(rl - p0 - 32) * CBS + m]) = f32x4{l[m], l[m + 1], l[m + 2], l[m + 3]};
            }
        }
        __syncthreads();
        // trailing update G_ij -= C_i C_j^T over the lower 32-blocks under the panel
        const int nbt = below / 32;
        for (int q = wave; q < nbt * (nbt + 1) / 2; q += 4) {
            int bi, bj;
            blk(q, bi, bj);
            f32x16 a = f32x16{};
#pragma unroll
            for (int k0 = 0; k0 < 32; k0 += 16)
                a = mma16(a, ld_frag(&Cb[(bi * 32 + lr) * CBS + k0 + lk]), ld_frag(&Cb[(bj * 32 + lr) * CBS + k0 + lk]));
            float *gb = G + (p0 + 32 + bi * 32) * GS + p0 + 32 + bj * 32;
#pragma unroll
            for (int t = 0; t < 16; ++t) gb[acc_row(lane, t) * GS + lr] -= a[t];
        }
        __syncthreads();
    }
    if (tid == 0) flags[b] = fail ? 1 : 0;
    if constexpr (FUSE) {
        if (tid == 0) sh_fail = fail ? 1 : 0;
        __syncthreads();
        if constexpr (KP == 64) {
            // lower-left block of C^-1: -C_11^-1 (C_10 C_00^-1).  Thread tid
            // takes column m = tid % 32 of rows i = tid / 32 + 8 u; the
            // diagonal blocks of Ci hold their zeros above the diagonal, so
            // the sums run over all 32 terms, fully unrolled (LDS reads in
            // batches, not one latency per term)
            const int m = tid & 31, i0 = tid >> 5;
            float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                const float c = Ci[k * CSS + m];
#pragma unroll
                for (int u = 0; u < 4; ++u) a[u] = fmaf(Cs[(32 + i0 + 8 * u) * CSS + k], c, a[u]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) Pm[(i0 + 8 * u) * 33 + m] = a[u];
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = 0.f;
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                const float pk = Pm[k * 33 + m];
#pragma unroll
                for (int u = 0; u < 4; ++u) a[u] = fmaf(Ci[(32 + i0 + 8 * u) * CSS + 32 + k], pk, a[u]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) Ci[(32 + i0 + 8 * u) * CSS + m] = -a[u];
            __syncthreads();
        }
        const bool dead = sh_fail != 0;
        // Q^T = C^-1 L1^T: wavefront w takes tokens 64 w .. 64 w + 63 (two
        // 32-token blocks), the L1 rows as stored (8 consecutive features of a
        // token per lane: an MFMA fragment as is)
        constexpr int NJB = KP / 32;
        f32x16 acc[NJB][2];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) acc[jb][0] = acc[jb][1] = f32x16{};
        const bf16 *lrow[2];
        bool tok[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int64_t t = 64 * wave + 32 * tb + lr;
            tok[tb] = t < n;
            lrow[tb] = Tb + (tok[tb] ? t : 0) * ldt;
        }
#pragma unroll
        for (int ks = 0; ks < KP / 16; ++ks) {
            const int m0 = ks * 16 + lk;
            bf16x8 bl[2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) bl[tb] = (tok[tb] && m0 < KC) ? ld_frag(lrow[tb] + m0) : bf16x8{};
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                if (NJB == 2 && jb == 0 && ks >= 2) continue;  // C^-1 is lower triangular
                const float *cr = Ci + (jb * 32 + lr) * CSS + m0;
                const f32x4 v0 = *reinterpret_cast<const f32x4 *>(cr);
                const f32x4 v1 = *reinterpret_cast<const f32x4 *>(cr + 4);
                bf16x8 hi, lo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = e < 4 ? v0[e] : v1[e - 4];
                    hi[e] = (bf16)v;
                    lo[e] = (bf16)(v - (float)hi[e]);
                }
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    acc[jb][tb] = mma16(acc[jb][tb], hi, bl[tb]);
                    acc[jb][tb] = mma16(acc[jb][tb], lo, bl[tb]);
                }
            }
        }
        // lane: token lr of the block, four consecutive features per group
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                if (!tok[tb]) continue;
                bf16 *dst = const_cast<bf16 *>(lrow[tb]);
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int j0 = jb * 32 + acc_row(lane, 4 * g4);
                    if (j0 >= KC) continue;
                    union { uint2 u; bf16 h[4]; } w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w.h[e] = dead ? bf16(0.f) : (bf16)acc[jb][tb][4 * g4 + e];
                    *reinterpret_cast<uint2 *>(dst + j0) = w.u;
                }
            }
    }
}

// Q_b = L1_b C^-T in place.  Each token row is spread over a group of G lanes
// (G = token_lanes), by 8-column chunks dealt round-robin: lane p of the group
// holds chunks p, p + G, p + 2G, ...  The forward substitution C q^T = l^T is
// taken column by column: step K scales q_K by 1 / C[K][K] in the lane that
// owns it, broadcasts it over the group (DPP), and every lane subtracts
// q_K C[m][K] from its columns m > K; with the chunks dealt round-robin the
// lanes keep equal shares of the shrinking trailing part, and chunks wholly
// at or left of K are skipped.  The factor, the same for every token, is
// staged in LDS (in the lanes' column order, the diagonal and everything above
// it zero, the reciprocal diagonal kept apart), so the updates need no
// masking.  64 G threads per workgroup, one token per group; rows of a failed
// instance become zero.
template <int KC>
__global__ __launch_bounds__(64 * token_lanes<KC>()) void q_apply_kernel(bf16 *__restrict__ T, int64_t ldt, int64_t off,
                                                                     int64_t n, const float *__restrict__ Ct,
                                                                     const int *__restrict__ flags) {
    constexpr int G = token_lanes<KC>();
    constexpr int PW = KC / G;   // columns per lane
    constexpr int NU = PW / 8;   // chunks per lane
    constexpr int NTH = 64 * G;
    constexpr int CH = stage_rows<KC>();
    static_assert(PW % 8 == 0 && KC % CH == 0, "columns per lane");
    __shared__ __align__(16) float Cs[CH * KC];  // Cs[K][lane-order column] = C[col][K] for col > K, else 0
    __shared__ float rd[KC];                      // 1 / C[K][K]
    const int tid = threadIdx.x;
    const int p = tid % G;
    const int64_t b = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 64 + tid / G;
    bf16 *const row = T + (b * n + (t < n ? t : n - 1)) * ldt + off;
    float x[PW];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        union { u32x4 u4; bf16 e[8]; } w;
        w.u4 = *reinterpret_cast<const u32x4 *>(row + 8 * (p + G * u));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * u + e] = (float)w.e[e];
    }
    const float *Cb = Ct + b * KC * KC;
    // one substitution step, K a compile-time constant (x is indexed by it)
    auto step = [&](auto Kc, const float *cs) __attribute__((always_inline)) {
        constexpr int K = decltype(Kc)::value;
        constexpr int cK = K / 8, PK = cK % G, IDX = 8 * (cK / G) + K % 8;
        const float sc = x[IDX] * rd[K];
        x[IDX] = p == PK ? sc : x[IDX];
        const float qk = group_bcast<G>(x[IDX], PK);
        const float *cr = cs + p * PW;
#pragma unroll
        for (int u = (K / 8) / G; u < NU; ++u) {
#pragma unroll
            for (int j0 = 0; j0 < 8; j0 += 4) {
                const f32x4 c = *reinterpret_cast<const f32x4 *>(cr + 8 * u + j0);
#pragma unroll
                for (int v = 0; v < 4; ++v) x[8 * u + j0 + v] = fmaf(-qk, c[v], x[8 * u + j0 + v]);
            }
        }
    };
    // rows [K0, K0 + CH) of the factor: staged in LDS, then their steps
    auto stage = [&](auto K0c) __attribute__((always_inline)) {
        constexpr int K0 = decltype(K0c)::value;
        if constexpr (K0 > 0) __syncthreads();  // the previous rows' reads are done
        for (int e = tid; e < CH * KC / 4; e += NTH) {
            const int Kl = (4 * e) / KC, pos = (4 * e) % KC;
            const int pp = pos / PW, uu = (pos % PW) / 8, jj = pos % 8;
            const int col = 8 * (pp + G * uu) + jj, K = K0 + Kl;
            f32x4 v = *reinterpret_cast<const f32x4 *>(Cb + K * KC + col);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (col + u == K) rd[K] = v[u];
                if (col + u <= K) v[u] = 0.f;
            }
            *reinterpret_cast<f32x4 *>(&Cs[Kl * KC + pos]) = v;
        }
        __syncthreads();
        unroll_seq<CH>([&](auto Klc) __attribute__((always_inline)) {
            constexpr int Kl = decltype(Klc)::value;
            step(std::integral_constant<int, K0 + Kl>{}, &Cs[Kl * KC]);
        });
    };
    unroll_seq<KC / CH>([&](auto Sc) __attribute__((always_inline)) {
        stage(std::integral_constant<int, decltype(Sc)::value * CH>{});
    });
    const bool dead = flags[b] != 0;
    if (t < n) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            union { u32x4 u4; bf16 e[8]; } w;
#pragma unroll
            for (int e = 0; e < 8; ++e) w.e[e] = dead ? bf16(0.f) : (bf16)x[8 * u + e];
            *reinterpret_cast<u32x4 *>(row + 8 * (p + G * u)) = w.u4;
        }
    }
}

// ------------------------------------------------------------- float32 path
// Correction ranks 16 and 32 (KP = kc): one workgroup per instance, every
// step that decides Q_b in float64, none of it serial beyond the k pivots.
//  1. G = L1_b^T L1_b: token chunks of 256 rows staged in LDS as stored;
//     each thread sums one 4 x 4 block of G over every (256 / blocks)-th
//     token of the chunk, and the partial G's are added in LDS, thread tid
//     then owning the entries tid + 256 u of G (row-major) (a product of two
//     float32 values is exact in float64).
//  2. Cholesky G + lambda I = C C^T, right-looking: column m of the trailing
//     matrix goes through LDS, one barrier per column.
//  3. Q_b = L1_b C^-T by forward substitution, one token per thread, the
//     rows of C read from LDS (one address per wavefront: broadcasts);
//     written in place over L1_b and, transposed, into Qt (zero for tokens
//     n..npad-1).
template <int KP>
__global__ __launch_bounds__(NT) void gram_q_f32_small_kernel(float *__restrict__ T, int64_t ldt, int64_t off,
                                                              int64_t n, int64_t npad, int kc_real, float lambda,
                                                              float *__restrict__ Qt, int *__restrict__ flags,
                                                              double *__restrict__ Cout) {
    static_assert(KP == 16 || KP == 32, "correction rank");
    constexpr int TC = 256;            // tokens per staged chunk
    constexpr int EPT = KP * KP / NT;  // entries of G per thread
    constexpr int V4 = KP / 4;         // 16-byte pieces of a token row
    __shared__ __align__(16) float Ls[TC * KP];
    __shared__ double Cs[KP][KP + 1];  // C, its diagonal replaced by 1 / C[i][i]
    __shared__ double colv[2][KP];
    __shared__ double diag[KP];
    __shared__ double sh_th;
    __shared__ int sh_fail;
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    float *const Lb = T + b * n * ldt + off;
    const int j = tid % KP;
    int iu[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) iu[u] = (tid + NT * u) / KP;
    // G by 4 x 4 blocks: thread (token group tg, block (bi, bj)) sums its block
    // over tokens tg, tg + TG, ... of each staged chunk, two 16-byte LDS reads
    // per token for 16 independent float64 FMAs; the TG partial G's meet in LDS
    constexpr int NB4 = KP / 4, NBLK = NB4 * NB4, TG = NT / NBLK;
    __shared__ double part[TG][KP * KP];
    const int blk = tid % NBLK, tg = tid / NBLK, bi = blk / NB4, bj = blk % NB4;
    double gb[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) gb[e] = 0.0;
    if (tid == 0) sh_fail = 0;

    // ---- 1. G
    for (int64_t t0 = 0; t0 < n; t0 += TC) {
        __syncthreads();  // the previous chunk's reads are done
        for (int e = tid; e < TC * V4; e += NT) {
            const int tok = e / V4, q = e % V4;
            const bool ok = t0 + tok < n;
            f32x4 v = *reinterpret_cast<const f32x4 *>(Lb + (ok ? t0 + tok : n - 1) * ldt + 4 * q);
            if (!ok) v = f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4 *>(&Ls[tok * KP + 4 * q]) = v;
        }
        __syncthreads();
        const int tc = (int)(n - t0 < TC ? n - t0 : TC);
#pragma unroll 4
        for (int t = tg; t < tc; t += TG) {
            const f32x4 ri = *reinterpret_cast<const f32x4 *>(&Ls[t * KP + 4 * bi]);
            const f32x4 rj = *reinterpret_cast<const f32x4 *>(&Ls[t * KP + 4 * bj]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int c = 0; c < 4; ++c) gb[4 * a + c] = fma((double)ri[a], (double)rj[c], gb[4 * a + c]);
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) part[tg][(4 * bi + a) * KP + 4 * bj + c] = gb[4 * a + c];
    __syncthreads();
    double g[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
        double sum = 0.0;
#pragma unroll
        for (int q = 0; q < TG; ++q) sum += part[q][tid + NT * u];
        g[u] = sum;
    }
    // lambda on the real diagonal, identity on the padding
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
        const int i = iu[u];
        if (i < kc_real && j < kc_real) g[u] += (i == j) ? (double)lambda : 0.0;
        else g[u] = (i == j) ? 1.0 : 0.0;
        if (i == j) diag[i] = g[u];
    }
    __syncthreads();
    if (tid == 0) {
        double dmax = 0.0;
        for (int i = 0; i < kc_real; ++i) dmax = dmax > diag[i] ? dmax : diag[i];
        // a pivot at or below the working precision times the largest
        // diagonal marks a numerically singular G (possible only for lambda = 0)
        sh_th = lambda > 0.f ? 0.0 : (double)KP * 2.3e-16 * dmax;
        if (!(dmax > 0.0)) sh_fail = 1;
    }
    // ---- 2. Cholesky, column m of the trailing matrix broadcast through colv[m & 1]
    for (int m = 0; m < KP; ++m) {
        double *cm = colv[m & 1];
#pragma unroll
        for (int u = 0; u < EPT; ++u)
            if (j == m) cm[iu[u]] = g[u];
        __syncthreads();
        double pk = cm[m];
        if (m < kc_real && !(pk > sh_th)) {
            if (tid == 0) sh_fail = 1;
            pk = 1.0;
        }
        const double d = sqrt(pk), rd = 1.0 / d, rp = rd * rd;
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int i = iu[u];
            if (j == m && i >= m) g[u] = (i == m) ? d : g[u] * rd;   // C[i][m]
            else if (j > m && i >= j) g[u] -= cm[i] * cm[j] * rp;   // trailing update
        }
    }
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
        const int i = iu[u];
        if (j > i) g[u] = 0.0;
        Cs[i][j] = (i == j) ? 1.0 / g[u] : g[u];
        if (Cout) Cout[(b * KP + i) * KP + j] = g[u];
    }
    __syncthreads();
    const bool dead = sh_fail != 0;
    if (tid == 0) flags[b] = dead ? 1 : 0;

    // ---- 3. q_t = C^-1 l_t, one token per thread (from the staged rows when
    // the instance was one chunk: npad <= TC then, and rows past n are zeros)
    float *const Qb = Qt + b * KP * npad;
    const bool staged = n <= TC && npad <= TC;
    for (int64_t t = tid; t < npad; t += NT) {
        double q[KP];
        const bool in = t < n;
#pragma unroll
        for (int v = 0; v < V4; ++v) {
            f32x4 x = staged ? *reinterpret_cast<const f32x4 *>(&Ls[t * KP + 4 * v])
                             : *reinterpret_cast<const f32x4 *>(Lb + (in ? t : n - 1) * ldt + 4 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) q[4 * v + e] = in ? (double)x[e] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            double s0 = q[i], s1 = 0.0;
#pragma unroll
            for (int c = 0; c < i; ++c) {
                if (c & 1) s1 = fma(-Cs[i][c], q[c], s1);
                else s0 = fma(-Cs[i][c], q[c], s0);
            }
            q[i] = dead ? 0.0 : (s0 + s1) * Cs[i][i];
        }
#pragma unroll
        for (int i = 0; i < KP; ++i) Qb[i * npad + t] = (float)q[i];
        if (in) {
#pragma unroll
            for (int v = 0; v < V4; ++v)
                *reinterpret_cast<f32x4 *>(Lb + t * ldt + 4 * v) =
                    f32x4{(float)q[4 * v], (float)q[4 * v + 1], (float)q[4 * v + 2], (float)q[4 * v + 3]};
        }
    }
}

// M'_b = Q_b^T X_b for float32 at correction ranks 16 and 32, on MFMA:
// workgroup (32 input features, instance b) forms the 32-feature slab of
// M'_b as one 32 x 32 block (correction rows i >= KP of it unused).  Its four
// wavefronts take the 16-token steps s = w, w + 4, ... (tokens past n are X's
// last row against Q_b's zero padding) and their partial blocks meet in LDS.
// A lane's X fragment is 8 tokens of one feature (consecutive lanes take
// consecutive features: one 128-byte segment of a token row per load); its Q
// fragment is 8 consecutive tokens of one row of Q_b^T as stored.  The single
// instance of a few hundred tokens is a latency problem: the scalar form (one
// thread per feature and token part) left 6 workgroups each a 64-token chain
// of 16 or 32 FMAs per token.
template <int KP>
__global__ __launch_bounds__(NT) void mprime_f32_mfma_kernel(const float *__restrict__ X, const float *__restrict__ Qt,
                                                             int64_t n, int64_t npad, int64_t c1,
                                                             float *__restrict__ Mp) {
    static_assert(KP == 16 || KP == 32, "correction rank");
    constexpr int NW = NT / 64;
    constexpr int G = 3;  // steps whose loads are requested together
    __shared__ float red[NW - 1][16][64];  // partial blocks of wavefronts 1.., [register][lane]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, hf = lane >> 5;
    const int64_t b = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * 32;
    // features past c1 read the last one, rows past KP the last row of Q_b^T:
    // neither is stored
    const float *const px = X + b * n * c1 + (c0 + lr < c1 ? c0 + lr : c1 - 1);
    const float *const pq = Qt + (b * KP + (lr < KP ? lr : KP - 1)) * npad + 8 * hf;
    const int S = (int)(npad / 16);
    f32x16 acc = f32x16{};
    for (int s0 = wave; s0 < S; s0 += NW * G) {
        f32x8 fx[G], fq[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int s = s0 + NW * u;
            const int64_t t0 = 16 * (int64_t)(s < S ? s : s0) + 8 * hf;  // a step past the end is skipped
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t t = t0 + e;
                fx[u][e] = px[(t < n ? t : n - 1) * c1];
            }
            fq[u] = ld_frag(pq + (t0 - 8 * hf));
        }
        // output row: feature c0 + acc_row; output column: correction row lr
#pragma unroll
        for (int u = 0; u < G; ++u)
            if (s0 + NW * u < S) acc = mma16(acc, fx[u], fq[u]);
    }
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t) red[wave - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wave != 0 || lr >= KP) return;
#pragma unroll
    for (int w = 0; w < NW - 1; ++w)
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] += red[w][t][lane];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t c = c0 + acc_row(lane, 4 * g);  // four consecutive features of row lr
        if (c < c1)
            *reinterpret_cast<f32x4 *>(Mp + (b * KP + lr) * c1 + c) =
                f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    }
}

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
                                                       bf16 *__restrict__ Mp, int64_t mp_rows, int mp_row0) {
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
            *reinterpret_cast<u32x4 *>(Mp + (b * mp_rows + mp_row0 + row) * c1 + f0 + 8 * c) =
                *reinterpret_cast<const u32x4 *>(ms + row * MS + 8 * c);
    }
}

}  // namespace

template <>
hipError_t launch_gram_q<bf16>(bf16 *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t, int kc_real,
                               int kc, float lambda, bf16 *, float *Ct, float *Gw, int *flags, double *Cout,
                               hipStream_t st) {
    if (B <= 0) return hipSuccess;
    const dim3 g1((unsigned)B), g2((unsigned)((n + 63) / 64), (unsigned)B);
    if (kc <= 64 && n <= NT) {
        // one launch: the workgroup of an instance holds all its tokens, so it
        // forms Q itself once C is done (no other workgroup reads its rows)
        switch (kc) {
#define DYRA_GQF(KC)                                                                                                 \
    case KC:                                                                                                         \
        hipLaunchKernelGGL((gram_chol_kernel<KC, false, true>), g1, dim3(NT), 0, st, T, ldt, off, n, kc_real, lambda,  \
                           Ct, Gw, flags, Cout);                                                                     \
        return hipGetLastError();
            DYRA_GQF(16) DYRA_GQF(32) DYRA_GQF(48) DYRA_GQF(64)
#undef DYRA_GQF
        default: return hipErrorInvalidValue;
        }
    }
    switch (kc) {
#define DYRA_GQ(KC)                                                                                                  \
    case KC:                                                                                                         \
        hipLaunchKernelGGL(gram_chol_kernel<KC>, g1, dim3(NT), 0, st, T, ldt, off, n, kc_real, lambda, Ct, Gw, flags, \
                           Cout);                                                                                    \
        hipLaunchKernelGGL(q_apply_kernel<KC>, g2, dim3(64 * token_lanes<KC>()), 0, st, T, ldt, off, n, Ct, flags);      \
        break;
        DYRA_GQ(16) DYRA_GQ(32) DYRA_GQ(48) DYRA_GQ(64) DYRA_GQ(80) DYRA_GQ(96) DYRA_GQ(112) DYRA_GQ(128)
        DYRA_GQ(144) DYRA_GQ(160) DYRA_GQ(176) DYRA_GQ(192) DYRA_GQ(208) DYRA_GQ(224) DYRA_GQ(240) DYRA_GQ(256)
#undef DYRA_GQ
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <>
hipError_t launch_gram_only<bf16>(const bf16 *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int kc_real, int kc,
                                  float lambda, float *G, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    switch (kc) {
#define DYRA_GO(KC)                                                                                                  \
    case KC:                                                                                                         \
        hipLaunchKernelGGL((gram_chol_kernel<KC, true>), dim3((unsigned)B), dim3(NT), 0, st, T, ldt, off, n, kc_real, \
                           lambda, nullptr, G, nullptr, nullptr);                                                    \
        break;
        DYRA_GO(80) DYRA_GO(96) DYRA_GO(112) DYRA_GO(128) DYRA_GO(144) DYRA_GO(160) DYRA_GO(176) DYRA_GO(192)
        DYRA_GO(208) DYRA_GO(224) DYRA_GO(240) DYRA_GO(256)
#undef DYRA_GO
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

size_t gram_workspace_floats(int kc) {
    const int kp = (kc + 31) / 32 * 32;
    return kp > 128 ? (size_t)kp * kp : 0;
}

template <>
hipError_t launch_gram_q<float>(float *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real,
                                int kc, float lambda, float *Qt, float *, float *, int *flags, double *Cout,
                                hipStream_t st) {
    if (B <= 0) return hipSuccess;
    if (kc < 1 || kc > 64) return hipErrorInvalidValue;
    if (kc == 16 || kc == 32) {
        if (kc == 16)
            hipLaunchKernelGGL(gram_q_f32_small_kernel<16>, dim3((unsigned)B), dim3(NT), 0, st, T, ldt, off, n, npad,
                               kc_real, lambda, Qt, flags, Cout);
        else
            hipLaunchKernelGGL(gram_q_f32_small_kernel<32>, dim3((unsigned)B), dim3(NT), 0, st, T, ldt, off, n, npad,
                               kc_real, lambda, Qt, flags, Cout);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(gram_q_f32_kernel, dim3((unsigned)B), dim3(NT), 0, st, T, ldt, off, n, npad, kc_real, kc,
                       lambda, Qt, flags, Cout);
    return hipGetLastError();
}

template <>
hipError_t launch_mprime<bf16>(const bf16 *X, const bf16 *T, int64_t ldt, int64_t off, const bf16 *, int64_t B,
                               int64_t n, int64_t, int64_t c1, int kc, bf16 *Mp, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    if (kc < 16 || kc % 16 != 0) return hipErrorInvalidValue;
    constexpr int CW = kMprimeFeatures;
    const dim3 grid((unsigned)((c1 + CW - 1) / CW), (unsigned)B);
    // correction ranks above 64 in passes of at most 64 rows of M'_b (X_b is
    // streamed once per pass)
    for (int r0 = 0; r0 < kc; r0 += 64) {
        const int w = kc - r0 < 64 ? kc - r0 : 64;
        switch (w) {
#define DYRA_MP(KC)                                                                                                   \
    case KC:                                                                                                          \
        hipLaunchKernelGGL((mprime_tr_kernel<KC, CW>), grid, dim3(NT), 0, st, X, T, ldt, off + r0, n, c1, Mp,          \
                           (int64_t)kc, r0);                                                                          \
        break;
            DYRA_MP(16) DYRA_MP(32) DYRA_MP(48) DYRA_MP(64)
#undef DYRA_MP
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <>
hipError_t launch_mprime<float>(const float *X, const float *, int64_t, int64_t, const float *Qt, int64_t B,
                                int64_t n, int64_t npad, int64_t c1, int kc, float *Mp, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    if (kc == 16 || kc == 32) {
        if (npad % 16 != 0) return hipErrorInvalidValue;
        const dim3 grid((unsigned)((c1 + 31) / 32), (unsigned)B);
        if (kc == 16)
            hipLaunchKernelGGL(mprime_f32_mfma_kernel<16>, grid, dim3(NT), 0, st, X, Qt, n, npad, c1, Mp);
        else
            hipLaunchKernelGGL(mprime_f32_mfma_kernel<32>, grid, dim3(NT), 0, st, X, Qt, n, npad, c1, Mp);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((mprime_kernel<float>), dim3((unsigned)((c1 + 255) / 256), (unsigned)B), dim3(NT), 0, st, X,
                       Qt, n, npad, c1, kc, Mp);
    return hipGetLastError();
}

}  // namespace dyra
