// Newton-Schulz SPD solve of the per-instance correction (gfx950).
//
// "DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
// DNNs", §2.4: for a large correction rank the r x r SPD system of Eq. 5 is
// solved with a Newton-Schulz iteration (matrix products) instead of the
// sequential Cholesky factorisation.  The path needs a factor F with
// F F^T = G^-1 (G = L1^T L1 + lambda I) so that Q = L1 F replaces L1 exactly
// as the Cholesky path's Q = L1 C^-T does; the coupled Newton-Schulz iteration
// gives the symmetric one, F = G^-1/2:
//     c = ||G||_F,  Y_0 = G / c,  Z_0 = I,
//     T_k = (3 I - Z_k Y_k) / 2,  Y_{k+1} = Y_k T_k,  Z_{k+1} = T_k Z_k,
//     F = Z_iters / sqrt(c).
// Every iterate is a polynomial in G (symmetric, commuting) in exact
// arithmetic; in float32 the products are formed as written (see
// mat_product).
//
//   ns_factor  workgroup per instance: G by MFMA over the instance's tokens
//              (chunks of 256, transposed through LDS as in gram_chol_kernel),
//              then the iteration on 64 x 64 float32 matrices held in LDS,
//              one 32 x 32 block of every product per wavefront
//              (v_mfma_f32_32x32x2_f32).  Correction indices past the real
//              rank get G = c I, which the iteration leaves at F = c^-1/2 I
//              without touching the real block.
//   ns_apply   workgroup per 64 tokens: Q = L1 F in place in T (float32
//              plans also write Q^T token-contiguous for their mprime).
// A rank-deficient G (lambda = 0) needs no special case: its null directions
// are null directions of L1, so whatever F does there, L1 F does not see it.
// Only a non-finite F (or G = 0) flags the instance, whose correction is then
// dropped.
#include "dyra_kernels.h"

#include "lanes.h"
#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;
constexpr int MS = 68;  // row stride (floats) of the 64 x 64 matrices in LDS (16-byte aligned rows)

typedef float Mat[64][MS];

// D = A B (64 x 64 float32 in LDS), one 32 x 32 block per wavefront: A's
// fragments along its rows, B's down its columns.  The product is formed
// exactly as written, never through B^T or a symmetrised copy: the coupled
// iteration is only stable when the rounding parts of Y and Z that break
// their symmetry are carried along (dropping them made float32 runs diverge
// within 20 steps at condition numbers near 1e3).  Ends with a barrier.
__device__ __forceinline__ void mat_product(const Mat &A, const Mat &B, Mat &D, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int k0 = 0; k0 < 64; k0 += 16) {
        f32x8 fb;
#pragma unroll
        for (int q = 0; q < 8; ++q) fb[q] = B[k0 + lk + q][wn * 32 + lr];
        acc = mma16(acc, ld_frag(&A[wm * 32 + lr][k0 + lk]), fb);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) D[wm * 32 + acc_row(lane, q)][wn * 32 + lr] = acc[q];
    __syncthreads();
}

template <typename E, int KC>
__global__ __launch_bounds__(NT) void ns_factor_kernel(const E *__restrict__ T, int64_t ldt, int64_t off, int64_t n,
                                                       int kc_real, float lambda, int iters, float *__restrict__ F,
                                                       int *__restrict__ flags) {
    constexpr int TT = NT;                          // tokens per Gram chunk
    constexpr int ST = TT + 16 / (int)sizeof(E);    // row stride (elements) of the transposed chunk
    __shared__ __align__(16) E Lt[64 * ST];         // [feature][token]
    __shared__ __align__(16) float M[4][64][MS];
    __shared__ float red[NT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t b = blockIdx.x;
    const E *Tb = T + b * n * ldt + off;
    for (int e = tid; e < (64 - KC) * ST; e += NT) Lt[KC * ST + e] = to_elem<E>(0.f);

    // ---- G = L1_b^T L1_b over all n tokens
    typedef typename Frag<E>::type Fr;
    f32x16 acc = f32x16{};
    for (int64_t c0 = 0; c0 < n; c0 += TT) {
        __syncthreads();  // the previous chunk's reads are done
        const int64_t t = c0 + tid;
        // the token's KC values as 16-byte loads, issued unconditionally (a
        // token past n rereads token n - 1 and is zeroed): guarded loads
        // compile to one branch and one full wait each
        constexpr int NV = KC * (int)sizeof(E) / 16;
        const E *row = Tb + (t < n ? t : n - 1) * ldt;
        u32x4 raw[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) raw[v] = *reinterpret_cast<const u32x4 *>(row + v * (16 / (int)sizeof(E)));
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            union { u32x4 u; E e[16 / sizeof(E)]; } w;
            w.u = raw[v];
#pragma unroll
            for (int q = 0; q < 16 / (int)sizeof(E); ++q)
                Lt[(v * (16 / (int)sizeof(E)) + q) * ST + tid] = t < n ? w.e[q] : to_elem<E>(0.f);
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < TT; kk += 16)
            acc = mma16(acc, ld_frag(Lt + (wm * 32 + lr) * ST + kk + lk), ld_frag(Lt + (wn * 32 + lr) * ST + kk + lk));
    }
    Mat &Y = M[0];
    Mat &Z = M[1];
    Mat &Tm = M[2];
    Mat &W = M[3];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int i = wm * 32 + acc_row(lane, q), j = wn * 32 + lr;
        Y[i][j] = (i < kc_real && j < kc_real) ? acc[q] + (i == j ? lambda : 0.f) : 0.f;
    }
    __syncthreads();
    // ---- c = ||G||_F over the real block
    float s = 0.f;
    for (int e = tid; e < 64 * 64; e += NT) {
        const float v = Y[e >> 6][e & 63];
        s = fmaf(v, v, s);
    }
    red[tid] = s;
    __syncthreads();
    for (int h = NT / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    const float c = sqrtf(red[0]);
    const float ic = c > 0.f ? 1.f / c : 0.f;
    for (int e = tid; e < 64 * 64; e += NT) {
        const int i = e >> 6, j = e & 63;
        const bool pad = i >= kc_real || j >= kc_real;
        Y[i][j] = pad ? (i == j ? 1.f : 0.f) : Y[i][j] * ic;  // padding: G = c I, so G / c = I
        Z[i][j] = i == j ? 1.f : 0.f;
    }
    __syncthreads();
    // ---- coupled iteration; the four buffers rotate: T = (3I - Z Y) / 2,
    // Y <- Y T (into W), Z <- T Z (into the old Y)
    int iy = 0, iz = 1, it = 2, iw = 3;
    for (int k = 0; k < iters; ++k) {
        mat_product(M[iz], M[iy], M[it], tid);
        for (int e = tid; e < 64 * 64; e += NT) {
            const int i = e >> 6, j = e & 63;
            M[it][i][j] = (i == j ? 1.5f : 0.f) - 0.5f * M[it][i][j];
        }
        __syncthreads();
        mat_product(M[iy], M[it], M[iw], tid);  // new Y
        mat_product(M[it], M[iz], M[iy], tid);  // new Z, over the old Y
        const int ny = iw, nz = iy, nw = iz;
        iy = ny;
        iz = nz;
        iw = nw;
    }
    // ---- F = Z / sqrt(c); a non-finite F or G = 0 flags the instance
    const float sc = c > 0.f ? rsqrtf(c) : 0.f;
    int bad = 0;
    float *Fb = F + b * KC * KC;
    for (int e = tid; e < KC * KC; e += NT) {
        const float v = M[iz][e / KC][e % KC] * sc;
        bad |= !isfinite(v);
        Fb[e] = v;
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) flags[b] = (bad || !(c > 0.f)) ? 1 : 0;
    (void)Tm;
    (void)W;
}

// Q = L1 F in place for 64 tokens of instance b (F = G^-1/2, symmetric up to
// rounding, so Q Q^T = L1 G^-1 L1^T); float32 plans
// also write Q^T token-contiguous into Qt ([B][KC][npad], zero past n).
// Rows of a flagged instance become zero.
template <typename E, int KC>
__global__ __launch_bounds__(NT) void ns_apply_kernel(E *__restrict__ T, int64_t ldt, int64_t off, int64_t n,
                                                      int64_t npad, const float *__restrict__ F,
                                                      const int *__restrict__ flags, float *__restrict__ Qt) {
    __shared__ float Ls[64][KC + 1];
    __shared__ float Fs[KC][KC + 1];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y, t0 = (int64_t)blockIdx.x * 64;
    E *Tb = T + b * n * ldt + off;
    for (int e = tid; e < KC * KC; e += NT) Fs[e / KC][e % KC] = F[b * KC * KC + e];
    for (int e = tid; e < 64 * KC; e += NT) {
        const int r = e / KC, m = e % KC;
        Ls[r][m] = t0 + r < n ? (float)Tb[(t0 + r) * ldt + m] : 0.f;
    }
    const bool dead = flags[b] != 0;
    __syncthreads();
    constexpr int CPT = KC / 4;  // columns per thread
    const int r = tid >> 2, c0 = (tid & 3) * CPT;
    const int64_t t = t0 + r;
    float q[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) q[u] = 0.f;
    for (int m = 0; m < KC; ++m) {
        const float l = Ls[r][m];
#pragma unroll
        for (int u = 0; u < CPT; ++u) q[u] = fmaf(l, Fs[m][c0 + u], q[u]);
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const float v = dead ? 0.f : q[u];
        if (t < n) Tb[t * ldt + c0 + u] = to_elem<E>(v);
        if (Qt && t < npad) Qt[(b * KC + c0 + u) * npad + t] = v;
    }
}

// ---------------------------------------------------------------------------
// Correction ranks above 64: the same iteration on kp x kp matrices (kp = kc
// rounded up to 32) kept in the workspace, each product formed for all
// instances in one launch.
//   gram     G_b (launch_gram_only, both triangles)
//   ns_init  workgroup per instance: c = ||G||_F over the real block,
//            Y = G / c (identity on the padding), Z = I
//   ns_prod  per step, two launches of a batched float32 MFMA product
//            (64 x 64 output tiles, K in slices of 32 staged through LDS,
//            B's slice stored transposed so both fragments read rows):
//            T = (3 I - Z Y) / 2 (the scaling fused into the store), then
//            Y' = Y T and Z' = T Z side by side in one launch
//   ns_apply_large  Q = L1 Z / sqrt(c) in place, each token row over a group
//            of lanes as in q_apply_kernel, Z staged in LDS in row pieces
constexpr int kPT = 64;   // output tile of ns_prod
constexpr int kPK = 32;   // K slice of ns_prod
constexpr int kPS = 36;   // LDS row stride (floats) of ns_prod's slices

__global__ __launch_bounds__(NT) void ns_init_kernel(float *__restrict__ Y, float *__restrict__ Z, int kp,
                                                     int kc_real, float *__restrict__ cs, int *__restrict__ flags) {
    __shared__ float red[NT];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    float *Yb = Y + b * kp * kp, *Zb = Z + b * kp * kp;
    float s = 0.f;
    for (int e = tid; e < kp * kp; e += NT) {
        const int i = e / kp, j = e - i * kp;
        if (i < kc_real && j < kc_real) s = fmaf(Yb[e], Yb[e], s);
    }
    red[tid] = s;
    __syncthreads();
    for (int h = NT / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    const float c = sqrtf(red[0]);
    const float ic = c > 0.f ? 1.f / c : 0.f;
    for (int e = tid; e < kp * kp; e += NT) {
        const int i = e / kp, j = e - i * kp;
        const bool pad = i >= kc_real || j >= kc_real;
        Yb[e] = pad ? (i == j ? 1.f : 0.f) : Yb[e] * ic;
        Zb[e] = i == j ? 1.f : 0.f;
    }
    if (tid == 0) {
        cs[b] = c;
        flags[b] = c > 0.f ? 0 : 1;
    }
}

// D_p = A_p B_p for product p = blockIdx.z (up to two per launch), every
// instance b = blockIdx.y, tile blockIdx.x; all [kp][kp] row-major, instance
// stride kp^2.  HALF3: D = (3 I - A B) / 2.
struct NsProd {
    const float *A[2];
    const float *B[2];
    float *D[2];
};

template <bool HALF3>
__global__ __launch_bounds__(NT) void ns_prod_kernel(NsProd pr, int kp) {
    __shared__ __align__(16) float As[kPT * kPS];
    __shared__ __align__(16) float Bt[kPT * kPS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int wm = wave >> 1, wn = wave & 1;
    const int z = blockIdx.z;
    const int64_t boff = (int64_t)blockIdx.y * kp * kp;
    const float *A = pr.A[z] + boff, *B = pr.B[z] + boff;
    float *D = pr.D[z] + boff;
    const int tn = kp / kPT;
    const int i0 = (blockIdx.x / tn) * kPT, j0 = (blockIdx.x % tn) * kPT;
    f32x16 acc = f32x16{};
    for (int k0 = 0; k0 < kp; k0 += kPK) {
        __syncthreads();  // the previous slice's reads are done
        // A rows i0.. (64 x 32) and B rows k0.. (32 x 64, stored transposed)
        for (int e = tid; e < kPT * kPK / 4; e += NT) {
            const int r = e / (kPK / 4), c4 = (e % (kPK / 4)) * 4;
            *reinterpret_cast<f32x4 *>(&As[r * kPS + c4]) =
                *reinterpret_cast<const f32x4 *>(A + (int64_t)(i0 + r) * kp + k0 + c4);
            const int rk = e / (kPT / 4), cj = (e % (kPT / 4)) * 4;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(B + (int64_t)(k0 + rk) * kp + j0 + cj);
#pragma unroll
            for (int u = 0; u < 4; ++u) Bt[(cj + u) * kPS + rk] = v[u];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kPK; kk += 16)
            acc = mma16(acc, ld_frag(&As[(wm * 32 + lr) * kPS + kk + lk]), ld_frag(&Bt[(wn * 32 + lr) * kPS + kk + lk]));
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int i = i0 + wm * 32 + acc_row(lane, t), j = j0 + wn * 32 + lr;
        D[(int64_t)i * kp + j] = HALF3 ? (i == j ? 1.5f : 0.f) - 0.5f * acc[t] : acc[t];
    }
}

// Q = L1 Z / sqrt(c) in place for 64 tokens of instance b, each token row over
// a group of lanes dealt 8-column chunks round-robin (lane p: chunks p, p + G,
// ...); step m broadcasts l_m over the group (DPP) and every lane adds
// l_m Z[m][j] to its columns j.  Z is staged in LDS in the lanes' column
// order, CH rows at a time.  A non-finite factor (or c = 0) flags the
// instance and zeroes its rows; every workgroup of the instance sees the same
// factor, and the first writes the flag.
template <int KC>
__global__ __launch_bounds__(64 * token_lanes<KC>()) void ns_apply_large_kernel(bf16 *__restrict__ T, int64_t ldt,
                                                                              int64_t off, int64_t n, int kp,
                                                                              const float *__restrict__ Z,
                                                                              const float *__restrict__ cs,
                                                                              int *__restrict__ flags) {
    constexpr int G = token_lanes<KC>();
    constexpr int PW = KC / G, NU = PW / 8, NTH = 64 * G;
    constexpr int CH = stage_rows<KC>();
    __shared__ __align__(16) float Zs[CH * KC];
    __shared__ int bad;
    const int tid = threadIdx.x;
    const int p = tid % G;
    const int64_t b = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 64 + tid / G;
    bf16 *const row = T + (b * n + (t < n ? t : n - 1)) * ldt + off;
    float l[PW], q[PW];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        union { u32x4 u4; bf16 e[8]; } w;
        w.u4 = *reinterpret_cast<const u32x4 *>(row + 8 * (p + G * u));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            l[8 * u + e] = (float)w.e[e];
            q[8 * u + e] = 0.f;
        }
    }
    const float c = cs[b];
    const float sc = c > 0.f ? rsqrtf(c) : 0.f;
    if (tid == 0) bad = !(c > 0.f);
    __syncthreads();  // set before any thread can raise it
    const float *Zb = Z + b * kp * kp;
    // one step, m a compile-time constant (l and q are indexed by it)
    auto step = [&](auto mc, const float *zrow) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        constexpr int cm = m / 8, PM = cm % G, IDX = 8 * (cm / G) + m % 8;
        const float lm = group_bcast<G>(l[IDX], PM);
        const float *zr = zrow + p * PW;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int j0 = 0; j0 < 8; j0 += 4) {
                const f32x4 zv = *reinterpret_cast<const f32x4 *>(zr + 8 * u + j0);
#pragma unroll
                for (int v = 0; v < 4; ++v) q[8 * u + j0 + v] = fmaf(lm, zv[v], q[8 * u + j0 + v]);
            }
        // the step's sums are formed here (otherwise every step's broadcast
        // and LDS reads are issued first and the sums left to the end)
#pragma unroll
        for (int j = 0; j < PW; ++j) asm volatile("" : "+v"(q[j]));
    };
    // rows [M0, M0 + CH) of Z: staged in LDS (finiteness checked), then their steps
    auto stage = [&](auto M0c) __attribute__((always_inline)) {
        constexpr int M0 = decltype(M0c)::value;
        if constexpr (M0 > 0) __syncthreads();
        bool nf = false;
        for (int e = tid; e < CH * KC / 4; e += NTH) {
            const int ml = (4 * e) / KC, pos = (4 * e) % KC;
            const int pp = pos / PW, uu = (pos % PW) / 8, jj = pos % 8;
            const int col = 8 * (pp + G * uu) + jj;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(Zb + (int64_t)(M0 + ml) * kp + col);
            nf = nf || !(isfinite(v[0]) && isfinite(v[1]) && isfinite(v[2]) && isfinite(v[3]));
            *reinterpret_cast<f32x4 *>(&Zs[ml * KC + pos]) = v;
        }
        if (nf) bad = 1;
        __syncthreads();
        unroll_seq<CH>([&](auto Mc) __attribute__((always_inline)) {
            constexpr int ml = decltype(Mc)::value;
            step(std::integral_constant<int, M0 + ml>{}, &Zs[ml * KC]);
        });
    };
    unroll_seq<KC / CH>([&](auto Sc) __attribute__((always_inline)) {
        stage(std::integral_constant<int, decltype(Sc)::value * CH>{});
    });
    __syncthreads();
    const bool dead = bad != 0;
    if (blockIdx.x == 0 && tid == 0) flags[b] = dead ? 1 : 0;
    if (t < n) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            union { u32x4 u4; bf16 e[8]; } w;
#pragma unroll
            for (int e = 0; e < 8; ++e) w.e[e] = dead ? bf16(0.f) : (bf16)(q[8 * u + e] * sc);
            *reinterpret_cast<u32x4 *>(row + 8 * (p + G * u)) = w.u4;
        }
    }
}

}  // namespace

size_t ns_workspace_floats(int64_t B, int kc) {
    if (kc <= 64) return (size_t)B * kc * kc;
    const int64_t kp = (kc + 31) / 32 * 32;
    return (size_t)B * (5 * kp * kp + 1);
}

template <typename E>
hipError_t launch_ns_solve(E *T, int64_t ldt, int64_t off, int64_t B, int64_t n, int64_t npad, int kc_real, int kc,
                           float lambda, int iters, float *F, int *flags, float *Qt, hipStream_t st,
                           const EventMark &mark) {
    if (B <= 0) return hipSuccess;
    hipError_t e;
    if (kc > 64) {
        if constexpr (sizeof(E) != 2) {
            return hipErrorInvalidValue;
        } else {
            // F holds Y0, Y1, Z0, Z1, T ([B][kp][kp] each) and c [B]
            const int kp = (kc + 31) / 32 * 32;
            const int64_t m = B * (int64_t)kp * kp;
            float *Yb[2] = {F, F + m}, *Zb[2] = {F + 2 * m, F + 3 * m}, *Tb = F + 4 * m, *cs = F + 5 * m;
            if ((e = launch_gram_only<E>(T, ldt, off, B, n, kc_real, kc, lambda, Yb[0], st)) != hipSuccess) return e;
            hipLaunchKernelGGL(ns_init_kernel, dim3((unsigned)B), dim3(NT), 0, st, Yb[0], Zb[0], kp, kc_real, cs,
                               flags);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            const unsigned tiles = (unsigned)((kp / kPT) * (kp / kPT));
            if (kp % kPT != 0) {
                // kp a multiple of 32 but not of 64: the products take one more
                // 32-row band; not built, so such ranks have no Newton-Schulz solve
                return hipErrorInvalidValue;
            }
            int cur = 0;
            for (int it = 0; it < iters; ++it) {
                NsProd p1{{Zb[cur], nullptr}, {Yb[cur], nullptr}, {Tb, nullptr}};
                hipLaunchKernelGGL(ns_prod_kernel<true>, dim3(tiles, (unsigned)B, 1), dim3(NT), 0, st, p1, kp);
                NsProd p2{{Yb[cur], Tb}, {Tb, Zb[cur]}, {Yb[1 - cur], Zb[1 - cur]}};
                hipLaunchKernelGGL(ns_prod_kernel<false>, dim3(tiles, (unsigned)B, 2), dim3(NT), 0, st, p2, kp);
                cur = 1 - cur;
            }
            if ((e = mark(hipGetLastError())) != hipSuccess) return e;
            const dim3 g2((unsigned)((n + 63) / 64), (unsigned)B);
            switch (kc) {
#define DYRA_NSL(KC)                                                                                             \
    case KC:                                                                                                     \
        hipLaunchKernelGGL((ns_apply_large_kernel<KC>), g2, dim3(64 * token_lanes<KC>()), 0, st, T, ldt, off, n, kp, \
                           Zb[cur], cs, flags);                                                                  \
        break;
                DYRA_NSL(128) DYRA_NSL(192) DYRA_NSL(256)
#undef DYRA_NSL
            default: return hipErrorInvalidValue;
            }
            return mark(hipGetLastError());
        }
    }
    const dim3 g2((unsigned)((npad + 63) / 64), (unsigned)B);
    switch (kc) {
#define DYRA_NS(KC)                                                                                             \
    case KC:                                                                                                    \
        hipLaunchKernelGGL((ns_factor_kernel<E, KC>), dim3((unsigned)B), dim3(NT), 0, st, T, ldt, off, n, kc_real, \
                           lambda, iters, F, flags);                                                            \
        if ((e = mark(hipGetLastError())) != hipSuccess) return e;                                              \
        hipLaunchKernelGGL((ns_apply_kernel<E, KC>), g2, dim3(NT), 0, st, T, ldt, off, n, npad, F, flags, Qt);  \
        break;
        DYRA_NS(16)
        DYRA_NS(32)
        DYRA_NS(48)
        DYRA_NS(64)
#undef DYRA_NS
    default: return hipErrorInvalidValue;
    }
    return mark(hipGetLastError());
}

template hipError_t launch_ns_solve<bf16>(bf16 *, int64_t, int64_t, int64_t, int64_t, int64_t, int, int, float, int,
                                          float *, int *, float *, hipStream_t, const EventMark &);
template hipError_t launch_ns_solve<float>(float *, int64_t, int64_t, int64_t, int64_t, int64_t, int, int, float, int,
                                           float *, int *, float *, hipStream_t, const EventMark &);

}  // namespace dyra
