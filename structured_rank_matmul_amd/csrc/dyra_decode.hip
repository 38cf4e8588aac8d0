// Dual-form (n < k) kernels of the DyRA forward path; see dyra_decode.h.
//
// "DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
// DNNs", Algorithm 1 Inference lines 10-13 and Eq. 5-7, evaluated through the
// push-through identity so that it stays defined when an instance has fewer
// tokens than the correction rank (token-by-token decode).  These shapes are
// bound by HBM: W_res and V_s are streamed once per call, 32 output columns
// per workgroup, and the small operands (X, T) are re-read from L2.
#include "dyra_decode.h"

#include <algorithm>

#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;
constexpr int kRowBlock = 64;  // rows (tokens) per workgroup, two 32-row MFMA blocks

constexpr int kMaxSplits = 4;  // split-K parts of the projection (16 measured slower overall)
constexpr int kMaxCorr = 64;    // largest padded correction rank

int decode_splits(int64_t c1) {
    int s = 1;
    while (s < kMaxSplits && c1 % (32 * 2 * s) == 0 && c1 / (2 * s) >= 256) s *= 2;
    return s;
}

int64_t rows_per_block(int64_t n) { return (kRowBlock / n) * n; }

struct DualLayout {
    size_t partial, T, coef, total;
    int splits;
};

DualLayout dual_layout(int64_t B, int64_t n, int64_t c1, int kw, int kc) {
    DualLayout L{};
    const int64_t N = B * n;
    const int64_t K1 = kw + kc;
    L.splits = decode_splits(c1);
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t off = 0;
    L.partial = off;
    off += al(sizeof(float) * (size_t)L.splits * N * K1);
    L.T = off;
    off += al(sizeof(float) * (size_t)N * K1);
    L.coef = off;
    off += al(sizeof(float) * (size_t)B * n * n);
    L.total = off;
    return L;
}

// Fragment of 8 consecutive elements from a float32 row, converted to E.
__device__ __forceinline__ bf16x8 frag_from_f32(const float *p, bf16) {
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(p + 4);
    bf16x8 r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
    r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
}
__device__ __forceinline__ f32x8 frag_from_f32(const float *p, float) { return ld_frag(p); }

constexpr int kUnroll = 4;     // 16-deep steps whose loads are requested together
constexpr int kUnrollRes = 4;  // the same for each of the two W_res register sets

// Fragment or zero, without a branch (the load itself always reads an address
// in range; lanes out of range point at a clamped one).
template <typename F> __device__ __forceinline__ F keep_if(bool ok, const F &f) { return ok ? f : F{}; }

// partial[s][row][col] = sum over the s-th split of c1 of X[row][k] Aext[col][k].
// Grid (K1/32 column blocks, splits, row blocks of 64).  Each of the four
// wavefronts takes a contiguous quarter of the split (its batched loads then
// cover whole 128-byte lines of each row), and the quarters meet in LDS.
template <typename E, bool TWO>
__global__ __launch_bounds__(NT) void decode_project_kernel(const E *__restrict__ X, const E *__restrict__ Aext,
                                                            int64_t N, int64_t c1, int K1, int splits,
                                                            float *__restrict__ partial) {
    __shared__ float red[NT / 64][kRowBlock * 32];  // each wavefront's partial [row][col]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int col0 = blockIdx.x * 32;
    const int s = blockIdx.y;
    const int64_t row0 = (int64_t)blockIdx.z * kRowBlock;
    const int64_t ks = c1 / splits;
    const int64_t kbeg = s * ks;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    const int col = col0 + lr;
    const bool col_ok = col < K1;
    const int64_t ra = row0 + lr, rb = row0 + 32 + lr;
    const bool a_ok = ra < N, b_ok = rb < N;
    const E *pb = Aext + (int64_t)(col_ok ? col : 0) * c1 + lk;
    const E *pa0 = X + (a_ok ? ra : row0) * c1 + lk;
    const E *pa1 = X + (b_ok ? rb : row0) * c1 + lk;
    typedef typename Frag<E>::type F;
    // kUnroll steps' loads are requested before their MFMAs; each wavefront
    // streams its own contiguous quarter of the split
    const int64_t q4 = ((ks + 63) / 64) * 16;
    const int64_t wb = kbeg + (wave * q4 < ks ? wave * q4 : ks);
    const int64_t we = kbeg + ((wave + 1) * q4 < ks ? (wave + 1) * q4 : ks);
    for (int64_t k0 = wb; k0 < we; k0 += 16 * kUnroll) {
        F fb[kUnroll], fa0[kUnroll], fa1[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t k = k0 + 16 * u;
            const bool kin = k < we;
            const int64_t kk = kin ? k : kbeg;
            fb[u] = keep_if(kin && col_ok, ld_frag(pb + kk));
            fa0[u] = keep_if(kin && a_ok, ld_frag(pa0 + kk));
            if constexpr (TWO) fa1[u] = keep_if(kin && b_ok, ld_frag(pa1 + kk));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            acc[0] = mma16(acc[0], fa0[u], fb[u]);
            if constexpr (TWO) acc[1] = mma16(acc[1], fa1[u], fb[u]);
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 16; ++t) red[wave][(h * 32 + acc_row(lane, t)) * 32 + lr] = acc[h][t];
    __syncthreads();
    for (int e = tid; e < kRowBlock * 32; e += NT) {
        const int r = e >> 5, c = e & 31;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) v += red[w][e];
        if (row0 + r < N && col0 + c < K1) partial[((int64_t)s * N + row0 + r) * K1 + col0 + c] = v;
    }
}

// One workgroup per instance: T rows = sum of the split partials; then
// C_b = K (K + lambda I)^-1 with K = L1_b L1_b^T (n x n) from the eigenpairs of
// K (cyclic Jacobi, float64, one thread).  K is formed in float64 from the
// float32 L1 values, so an exact rank deficiency shows as eigenvalues at the
// float64 rounding level; at lambda = 0 eigenvalues below n * 1e-12 * max
// count as zero, giving the projector onto range(L1_b).
template <typename E>
__global__ __launch_bounds__(NT) void decode_coef_kernel(const float *__restrict__ partial, int64_t N, int64_t n,
                                                         int K1, int kw, int k_real, int splits, float lambda,
                                                         float *__restrict__ T, float *__restrict__ coef,
                                                         int *__restrict__ flags) {
    __shared__ double K[16][16];
    __shared__ double V[16][16];
    __shared__ float Ls[16][kMaxCorr + 1];  // the instance's L1 rows (the Gram's operand)
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t r0 = b * n;
    // every split's value of kEB elements per thread requested before the
    // first add (one load latency per batch; past the end, element 0 and
    // split 0 are reread and dropped)
    constexpr int kEB = 4;
    const int64_t total = n * K1;
    for (int64_t e0 = tid; e0 < total; e0 += (int64_t)NT * kEB) {
        float v[kEB][kMaxSplits];
#pragma unroll
        for (int j = 0; j < kEB; ++j) {
            const int64_t e = e0 + (int64_t)j * NT < total ? e0 + (int64_t)j * NT : 0;
            const int64_t i = e / K1, c = e - i * K1;
#pragma unroll
            for (int q = 0; q < kMaxSplits; ++q)
                v[j][q] = partial[((int64_t)(q < splits ? q : 0) * N + r0 + i) * K1 + c];
        }
#pragma unroll
        for (int j = 0; j < kEB; ++j) {
            const int64_t e = e0 + (int64_t)j * NT;
            if (e >= total) continue;
            const int64_t i = e / K1, c = e - i * K1;
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < kMaxSplits; ++q) s += q < splits ? v[j][q] : 0.f;
            T[(r0 + i) * K1 + c] = s;
            if (c >= kw) Ls[i][c - kw] = s;
        }
    }
    __syncthreads();
    const int nn = (int)n;
    // one Gram element per wavefront at a time: lanes over the correction
    // columns (k_real <= 64), then a butterfly sum
    const int lane = tid & 63, wave = tid >> 6;
    for (int e = wave; e < nn * nn; e += NT / 64) {
        const int i = e / nn, j = e - (e / nn) * nn;
        double s = lane < k_real ? (double)Ls[i][lane] * (double)Ls[j][lane] : 0.0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
        if (lane == 0) K[i][j] = s;
    }
    __syncthreads();
    if (tid == 0) {
        for (int i = 0; i < nn; ++i)
            for (int j = 0; j < nn; ++j) V[i][j] = (i == j) ? 1.0 : 0.0;
        for (int sweep = 0; sweep < 50; ++sweep) {
            double off = 0.0, tot = 0.0;
            for (int i = 0; i < nn; ++i)
                for (int j = 0; j < nn; ++j) {
                    tot += K[i][j] * K[i][j];
                    if (i != j) off += K[i][j] * K[i][j];
                }
            if (off <= 1e-30 * tot || off == 0.0) break;
            for (int p = 0; p < nn - 1; ++p)
                for (int q = p + 1; q < nn; ++q) {
                    const double apq = K[p][q];
                    if (apq == 0.0) continue;
                    const double theta = (K[q][q] - K[p][p]) / (2.0 * apq);
                    const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
                    const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
                    for (int m = 0; m < nn; ++m) {  // K <- K J (columns p, q)
                        const double kp = K[m][p], kq = K[m][q];
                        K[m][p] = c * kp - s * kq;
                        K[m][q] = s * kp + c * kq;
                    }
                    for (int m = 0; m < nn; ++m) {  // K <- J^T K (rows p, q)
                        const double kp = K[p][m], kq = K[q][m];
                        K[p][m] = c * kp - s * kq;
                        K[q][m] = s * kp + c * kq;
                    }
                    for (int m = 0; m < nn; ++m) {  // V <- V J
                        const double vp = V[m][p], vq = V[m][q];
                        V[m][p] = c * vp - s * vq;
                        V[m][q] = s * vp + c * vq;
                    }
                }
        }
        double mu_max = 0.0;
        for (int i = 0; i < nn; ++i) mu_max = fmax(mu_max, K[i][i]);
        const double tol = (double)nn * 1e-12 * mu_max;
        double f[16];
        for (int i = 0; i < nn; ++i) {
            const double mu = fmax(K[i][i], 0.0);
            if (lambda > 0.f) f[i] = mu / (mu + (double)lambda);
            else f[i] = (mu > tol && mu > 0.0) ? 1.0 : 0.0;
        }
        float *Cb = coef + b * n * n;
        for (int i = 0; i < nn; ++i)
            for (int j = 0; j < nn; ++j) {
                double s = 0.0;
                for (int m = 0; m < nn; ++m) s += V[i][m] * f[m] * V[j][m];
                Cb[i * nn + j] = (float)s;
            }
        flags[b] = 0;
    }
}

// Y[rows][col0..col0+32) = T_s V_s^T + bias + alpha blockdiag(C_b) (X W_res)
// (§2.4's fused output with bias and correction weight alpha).  Grid (c2/32,
// row blocks of whole instances).  Each wavefront takes a contiguous quarter of
// both contractions (measured 11-15 % faster per decode step than dealing the
// 16-deep steps round-robin, whose loads touch 32 bytes of 32 lines each), and
// the quarters are reduced in LDS.
template <typename E, bool TWO>
__global__ __launch_bounds__(NT) void decode_output_kernel(const E *__restrict__ X, const float *__restrict__ T,
                                                           const float *__restrict__ coef,
                                                           const E *__restrict__ Vs, const E *__restrict__ Wres_t,
                                                           int64_t N, int64_t n, int64_t c1, int64_t c2, int K1,
                                                           int kw, int64_t rows_blk, const E *__restrict__ bias,
                                                           float alpha, E *__restrict__ Y) {
    __shared__ float part[NT / 64][kRowBlock * 32];  // each wavefront's partial [row][col]
    __shared__ float Zs[kRowBlock][33];              // X W_res of the block, summed
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int64_t col0 = (int64_t)blockIdx.x * 32;
    const int64_t row0 = (int64_t)blockIdx.y * rows_blk;
    const int64_t row_end = (row0 + rows_blk < N) ? row0 + rows_blk : N;
    typedef typename Frag<E>::type F;
    const int64_t col = col0 + lr;
    const bool col_ok = col < c2;
    const int64_t ra = row0 + lr, rb = row0 + 32 + lr;
    const bool a_ok = ra < row_end, b_ok = rb < row_end;
    f32x16 z0 = f32x16{}, z1 = f32x16{}, s0 = f32x16{}, s1 = f32x16{};
    // both contractions request kUnroll steps' loads of the streamed W_res /
    // V_s columns before their MFMAs
    const int64_t colc = col_ok ? col : 0, rac = a_ok ? ra : row0, rbc = b_ok ? rb : row0;
    {
        // W_res is the long stream: two register sets, the next batch's loads
        // requested before the current batch's MFMAs.  Loads are unconditional
        // (steps past c1 reread step 0); the zeroing happens at the MFMA, so a
        // batch's data is waited for only there.
        constexpr int U = kUnrollRes;
        const E *pb = Wres_t + colc * c1 + lk, *pa0 = X + rac * c1 + lk, *pa1 = X + rbc * c1 + lk;
        // each wavefront streams its own contiguous quarter of c1
        const int64_t q4 = ((c1 + 63) / 64) * 16;
        const int64_t kb = wave * q4 < c1 ? wave * q4 : c1;
        const int64_t ke = (wave + 1) * q4 < c1 ? (wave + 1) * q4 : c1;
        auto load = [&](int64_t k0, F (&fb)[U], F (&fa0)[U], F (&fa1)[U]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t k = k0 + 16 * u;
                const int64_t kk = k < ke ? k : 0;
                fb[u] = ld_frag(pb + kk);
                fa0[u] = ld_frag(pa0 + kk);
                if constexpr (TWO) fa1[u] = ld_frag(pa1 + kk);
            }
        };
        auto mma = [&](int64_t k0, const F (&fb)[U], const F (&fa0)[U], const F (&fa1)[U])
                       __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool kin = k0 + 16 * u < ke;
                const F b = keep_if(kin && col_ok, fb[u]);
                z0 = mma16(z0, keep_if(a_ok, fa0[u]), b);
                if constexpr (TWO) z1 = mma16(z1, keep_if(b_ok, fa1[u]), b);
            }
        };
        F ab[U], a0[U], a1[U], bb[U], b0[U], b1[U];
        constexpr int64_t BS = 16 * U;  // K advance of one batch
        int64_t k0 = kb;
        load(k0, ab, a0, a1);
        __builtin_amdgcn_sched_barrier(0);
        for (; k0 < ke; k0 += 2 * BS) {
            load(k0 + BS, bb, b0, b1);
            mma(k0, ab, a0, a1);
            __builtin_amdgcn_sched_barrier(0);
            load(k0 + 2 * BS, ab, a0, a1);
            mma(k0 + BS, bb, b0, b1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    {
        const E *pb = Vs + colc * kw + lk;
        const float *pa0 = T + rac * K1 + lk, *pa1 = T + rbc * K1 + lk;
        const int q4 = ((kw + 63) / 64) * 16;
        const int vb = wave * q4 < kw ? wave * q4 : kw, ve = (wave + 1) * q4 < kw ? (wave + 1) * q4 : kw;
        for (int k0 = vb; k0 < ve; k0 += 16 * kUnroll) {
            F fb[kUnroll], fa0[kUnroll], fa1[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int k = k0 + 16 * u;
                const bool kin = k < ve;
                const int kk = kin ? k : 0;
                fb[u] = keep_if(kin && col_ok, ld_frag(pb + kk));
                fa0[u] = keep_if(kin && a_ok, frag_from_f32(pa0 + kk, E{}));
                if constexpr (TWO) fa1[u] = keep_if(kin && b_ok, frag_from_f32(pa1 + kk, E{}));
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                s0 = mma16(s0, fa0[u], fb[u]);
                if constexpr (TWO) s1 = mma16(s1, fa1[u], fb[u]);
            }
        }
    }
    // Z = X W_res summed over the wavefronts' steps into Zs
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int r = acc_row(lane, t);
        part[wave][r * 32 + lr] = z0[t];
        part[wave][(32 + r) * 32 + lr] = z1[t];
    }
    __syncthreads();
    for (int e = tid; e < kRowBlock * 32; e += NT) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) v += part[w][e];
        Zs[e >> 5][e & 31] = v;
    }
    __syncthreads();
    // S = T_s V_s^T partials in the same buffer (its Z reads are done)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int r = acc_row(lane, t);
        part[wave][r * 32 + lr] = s0[t];
        part[wave][(32 + r) * 32 + lr] = s1[t];
    }
    __syncthreads();
    for (int e = tid; e < kRowBlock * 32; e += NT) {
        const int r = e >> 5, c = e & 31;
        const int64_t row = row0 + r;
        if (row >= row_end || col0 + c >= c2) continue;
        float sv = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) sv += part[w][e];
        const int64_t b = row / n;
        const int i = (int)(row - b * n);
        const int rb0 = (int)(b * n - row0);
        const float *Cb = coef + b * n * n;
        float z = 0.f;
        for (int j = 0; j < (int)n; ++j) z += Cb[i * n + j] * Zs[rb0 + j][c];
        float v = sv + alpha * z;
        if (bias) v += (float)bias[col0 + c];
        Y[row * c2 + col0 + c] = to_elem<E>(v);
    }
}

}  // namespace

size_t decode_workspace_bytes(int64_t B, int64_t n, int64_t c1, int kw, int kc) {
    return dual_layout(B, n, c1, kw, kc).total;
}

template <typename E> hipError_t launch_decode_project(const DecodeArgs<E> &a, hipStream_t st) {
    const DualLayout L = dual_layout(a.B, a.n, a.c1, a.kw, a.kc);
    const int64_t N = a.B * a.n;
    const int K1 = a.kw + a.kc;
    dim3 grid((unsigned)((K1 + 31) / 32), (unsigned)L.splits, (unsigned)((N + kRowBlock - 1) / kRowBlock));
    if (N > 32)
        hipLaunchKernelGGL((decode_project_kernel<E, true>), grid, dim3(NT), 0, st, a.X, a.Aext, N, a.c1, K1,
                           L.splits, (float *)(a.ws + L.partial));
    else
        hipLaunchKernelGGL((decode_project_kernel<E, false>), grid, dim3(NT), 0, st, a.X, a.Aext, N, a.c1, K1,
                           L.splits, (float *)(a.ws + L.partial));
    return hipGetLastError();
}

template <typename E> hipError_t launch_decode_coef(const DecodeArgs<E> &a, hipStream_t st) {
    const DualLayout L = dual_layout(a.B, a.n, a.c1, a.kw, a.kc);
    const int64_t N = a.B * a.n;
    hipLaunchKernelGGL((decode_coef_kernel<E>), dim3((unsigned)a.B), dim3(NT), 0, st,
                       (const float *)(a.ws + L.partial), N, a.n, a.kw + a.kc, a.kw, a.k_real, L.splits, a.lambda,
                       (float *)(a.ws + L.T), (float *)(a.ws + L.coef), a.flags);
    return hipGetLastError();
}

template <typename E> hipError_t launch_decode_output(const DecodeArgs<E> &a, hipStream_t st) {
    const DualLayout L = dual_layout(a.B, a.n, a.c1, a.kw, a.kc);
    const int64_t N = a.B * a.n;
    const int64_t rb = rows_per_block(a.n);
    dim3 grid((unsigned)((a.c2 + 31) / 32), (unsigned)((N + rb - 1) / rb));
    // the second 32-row MFMA block only when some row block has rows there
    if (std::min<int64_t>(rb, N) > 32)
        hipLaunchKernelGGL((decode_output_kernel<E, true>), grid, dim3(NT), 0, st, a.X,
                           (const float *)(a.ws + L.T), (const float *)(a.ws + L.coef), a.Vs, a.Wres_t, N, a.n,
                           a.c1, a.c2, a.kw + a.kc, a.kw, rb, a.bias, a.alpha, a.Y);
    else
        hipLaunchKernelGGL((decode_output_kernel<E, false>), grid, dim3(NT), 0, st, a.X,
                           (const float *)(a.ws + L.T), (const float *)(a.ws + L.coef), a.Vs, a.Wres_t, N, a.n,
                           a.c1, a.c2, a.kw + a.kc, a.kw, rb, a.bias, a.alpha, a.Y);
    return hipGetLastError();
}

template hipError_t launch_decode_project<bf16>(const DecodeArgs<bf16> &, hipStream_t);
template hipError_t launch_decode_coef<bf16>(const DecodeArgs<bf16> &, hipStream_t);
template hipError_t launch_decode_output<bf16>(const DecodeArgs<bf16> &, hipStream_t);
template hipError_t launch_decode_project<float>(const DecodeArgs<float> &, hipStream_t);
template hipError_t launch_decode_coef<float>(const DecodeArgs<float> &, hipStream_t);
template hipError_t launch_decode_output<float>(const DecodeArgs<float> &, hipStream_t);

}  // namespace dyra
