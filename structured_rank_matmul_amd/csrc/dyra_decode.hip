// Dual-form (n < k) kernels of the DyRA forward path; see dyra_decode.h.
//
// "DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
// DNNs", Algorithm 1 Inference lines 10-13 and Eq. 5-7, evaluated through the
// push-through identity so that it stays defined when an instance has fewer
// tokens than the correction rank (token-by-token decode).  These shapes are
// bound by HBM: W_res and V_s are streamed once per call (W_res by
// decode_z_kernel in split-K parts of 64 output columns, V_s by
// decode_output_kernel, 32 columns per workgroup), and the small operands
// (X, T) are re-read from L2.
#include "dyra_decode.h"

#include <algorithm>

#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;
constexpr int kRowBlock = 64;  // rows (tokens) per workgroup, two 32-row MFMA blocks

constexpr int kMaxSplits = 8;  // split-K parts of the projection (16 measured slower overall)
constexpr int kMaxCorr = 256;   // largest padded correction rank

int decode_splits(int64_t c1) {
    int s = 1;
    // eight parts only for long contractions (c1 >= 8192: the down projection,
    // whose 34 column blocks leave most compute units idle at four)
    while (s < kMaxSplits && c1 % (32 * 2 * s) == 0 && c1 / (2 * s) >= (s < 4 ? 256 : 1024)) s *= 2;
    return s;
}

int64_t rows_per_block(int64_t n) { return (kRowBlock / n) * n; }

// Split-K parts of the W_res stream (decode_z_kernel): enough 64-column
// workgroups to cover the compute units about twice, each wavefront's share
// of a split at least 128 deep and a whole number of 16-deep steps.
constexpr int kZCols = 64;         // output columns per decode_z workgroup
constexpr int kZTargetBlocks = 512;
int z_splits(int64_t c1, int64_t c2) {
    const int64_t cb = (c2 + kZCols - 1) / kZCols;
    int s = 1;
    while (s < 16 && cb * 2 * s <= kZTargetBlocks && c1 % (64 * 2 * s) == 0 && c1 / (2 * s) >= 512) s *= 2;
    return s;
}

struct DualLayout {
    size_t partial, T, coef, zpart, Xt, Tt, total;
    int splits, zsplits;
};

DualLayout dual_layout(int64_t B, int64_t n, int64_t c1, int64_t c2, int kw, int kc) {
    DualLayout L{};
    const int64_t N = B * n;
    const int64_t K1 = kw + kc;
    L.splits = decode_splits(c1);
    L.zsplits = z_splits(c1, c2);
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t off = 0;
    L.partial = off;
    off += al(sizeof(float) * (size_t)L.splits * N * K1);
    L.T = off;
    off += al(sizeof(float) * (size_t)N * K1);
    L.coef = off;
    off += al(sizeof(float) * (size_t)B * n * n);
    L.zpart = off;
    off += al(sizeof(float) * (size_t)L.zsplits * N * c2);
    // X and T_s in MFMA fragment order (frag_index), whole 32-row blocks, at
    // most 4 bytes per element
    const size_t rows32 = (size_t)((N + 31) / 32) * 32;
    L.Xt = off;
    off += al(sizeof(float) * rows32 * (size_t)c1);
    L.Tt = off;
    off += al(sizeof(float) * rows32 * (size_t)kw);
    L.total = off;
    return L;
}

// Element (row, col) of a [rows][K] matrix stored in MFMA fragment order: the
// 32 x 16 block (row block, 16-deep step) is 512 consecutive elements, lane
// 32 h + r holding row r of the block, columns 8 h .. 8 h + 7 of the step.
// A wavefront that walks the contraction of one row block then reads one
// contiguous run, each lane's 8 elements already an MFMA operand.
__device__ __forceinline__ int64_t frag_index(int64_t row, int64_t col, int64_t K) {
    return ((row >> 5) * (K >> 4) + (col >> 4)) * 512 + (((col >> 3) & 1) * 32 + (row & 31)) * 8 + (col & 7);
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
                                                            float *__restrict__ partial, E *__restrict__ Xt) {
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
    // [A_s | P_L] in fragment order: the 32-column block's run, 1 KB per load
    const E *pb = Aext + (int64_t)(col0 / 32) * 32 * c1 + 8 * lane;
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
            fb[u] = keep_if(kin && col_ok, ld_frag(pb + 32 * kk));
            fa0[u] = keep_if(kin && a_ok, ld_frag(pa0 + kk));
            if constexpr (TWO) fa1[u] = keep_if(kin && b_ok, ld_frag(pa1 + kk));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            acc[0] = mma16(acc[0], fa0[u], fb[u]);
            if constexpr (TWO) acc[1] = mma16(acc[1], fa1[u], fb[u]);
        }
        // X also goes to the workspace in fragment order for the W_res stream
        // (decode_z_kernel): each 16-deep step by one column block (dealt
        // round-robin, so the stores spread over the grid), every element once
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t k = k0 + 16 * u;
            if (k >= we || (k >> 4) % gridDim.x != blockIdx.x) continue;
            if (a_ok) *reinterpret_cast<F *>(Xt + frag_index(ra, k + lk, c1)) = fa0[u];
            if (TWO && b_ok) *reinterpret_cast<F *>(Xt + frag_index(rb, k + lk, c1)) = fa1[u];
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
                                                         float *__restrict__ T, E *__restrict__ Tt, float *__restrict__ coef,
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
            else Tt[frag_index(r0 + i, c, kw)] = to_elem<E>(s);
        }
    }
    __syncthreads();
    const int nn = (int)n;
    // one Gram element per wavefront at a time: lanes over the correction
    // columns (k_real <= 256, in passes of 64), then a butterfly sum
    const int lane = tid & 63, wave = tid >> 6;
    for (int e = wave; e < nn * nn; e += NT / 64) {
        const int i = e / nn, j = e - (e / nn) * nn;
        double s = 0.0;
        for (int c = lane; c < k_real; c += 64) s += (double)Ls[i][c] * (double)Ls[j][c];
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

// One workgroup per instance for 16 < n <= 64 tokens with lambda = 0 (fewer
// tokens than the correction rank): T rows = sum of the split partials, and
// C_b = the orthogonal projector onto range(L1_b), the lambda -> 0 limit of
// L1 L1^T (L1 L1^T + lambda I)^-1.  K = L1_b L1_b^T is formed in float64 from
// the float32 L1 values and factored by a Cholesky with diagonal pivoting,
// which stops at the first remaining diagonal at or below n * 1e-12 times the
// largest diagonal of K: the factor's columns then span range(K) = range(L1_b)
// and their count is its numerical rank.  Full rank (the generic case, L1_b
// has independent rows) gives C_b = I exactly; a deficient rank gives
// C_b = F (F^T F)^-1 F^T for the factor's columns F (Gauss-Jordan inverse of
// the small SPD F^T F, float64).
constexpr int kWideTokens = 64;

template <typename E>
__global__ __launch_bounds__(NT) void decode_coef_wide_kernel(const float *__restrict__ partial, int64_t N,
                                                              int64_t n, int K1, int kw, int k_real, int splits,
                                                              float *__restrict__ T, E *__restrict__ Tt, float *__restrict__ coef,
                                                              int *__restrict__ flags) {
    constexpr int KS = kMaxCorr + 1;
    constexpr int MS = kWideTokens + 1;
    // the L1 rows (float32) while K is formed, afterwards the product W = F M^-1
    __shared__ __align__(16) char buf[kWideTokens * KS * sizeof(float)];
    __shared__ double Km[kWideTokens][MS];  // K, then F^T F and its inverse
    __shared__ double Fm[kWideTokens][MS];  // pivoted factor, one column per accepted step
    __shared__ int done[kWideTokens];
    __shared__ int sh_p, sh_rank;
    __shared__ double sh_d, sh_tol;
    float(*Ls)[KS] = reinterpret_cast<float(*)[KS]>(buf);
    double(*Wm)[MS] = reinterpret_cast<double(*)[MS]>(buf);
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t r0 = b * n;
    const int nn = (int)n;
    // ---- T rows and L1 (split partials summed)
    const int64_t total = n * K1;
    for (int64_t e = tid; e < total; e += NT) {
        const int64_t i = e / K1, c = e - i * K1;
        float s = 0.f;
        for (int q = 0; q < splits; ++q) s += partial[((int64_t)q * N + r0 + i) * K1 + c];
        T[(r0 + i) * K1 + c] = s;
        if (c >= kw) Ls[i][c - kw] = s;
        else Tt[frag_index(r0 + i, c, kw)] = to_elem<E>(s);
    }
    if (tid < kWideTokens) done[tid] = 0;
    __syncthreads();
    // ---- K = L1 L1^T, float64 (lower triangle computed, mirrored)
    for (int e = tid; e < nn * nn; e += NT) {
        const int i = e / nn, j = e - i * nn;
        if (j > i) continue;
        double s = 0.0;
        for (int c = 0; c < k_real; ++c) s += (double)Ls[i][c] * (double)Ls[j][c];
        Km[i][j] = s;
        Km[j][i] = s;
    }
    __syncthreads();
    if (tid == 0) {
        double d = 0.0;
        for (int i = 0; i < nn; ++i) d = fmax(d, Km[i][i]);
        sh_tol = (double)nn * 1e-12 * d;
        sh_rank = 0;
    }
    __syncthreads();
    // ---- Cholesky with diagonal pivoting, right-looking
    for (int s = 0; s < nn; ++s) {
        if (tid == 0) {
            int p = -1;
            double d = sh_tol;
            for (int i = 0; i < nn; ++i)
                if (!done[i] && Km[i][i] > d) {
                    d = Km[i][i];
                    p = i;
                }
            sh_p = p;
            sh_d = d;
        }
        __syncthreads();
        const int p = sh_p;
        if (p < 0) break;
        const double sq = sqrt(sh_d), rs = 1.0 / sq;
        if (tid < nn) Fm[tid][s] = done[tid] ? 0.0 : (tid == p ? sq : Km[tid][p] * rs);
        __syncthreads();
        for (int e = tid; e < nn * nn; e += NT) {
            const int i = e / nn, j = e - i * nn;
            Km[i][j] -= Fm[i][s] * Fm[j][s];
        }
        if (tid == 0) {
            done[p] = 1;
            sh_rank = s + 1;
        }
        __syncthreads();
    }
    const int rank = sh_rank;
    float *Cb = coef + b * n * n;
    if (rank == nn || rank == 0) {
        // independent token rows: the projector is the identity; no rows: zero
        for (int e = tid; e < nn * nn; e += NT) Cb[e] = (rank == nn && e / nn == e % nn) ? 1.f : 0.f;
    } else {
        // M = F^T F (rank x rank), then its inverse in place (Gauss-Jordan,
        // SPD: no pivoting), W = F M^-1, C_b = W F^T
        for (int e = tid; e < rank * rank; e += NT) {
            const int a = e / rank, c = e - a * rank;
            double s = 0.0;
            for (int i = 0; i < nn; ++i) s += Fm[i][a] * Fm[i][c];
            Km[a][c] = s;
        }
        __syncthreads();
        for (int q = 0; q < rank; ++q) {
            const double piv = Km[q][q];
            __syncthreads();
            // row q scaled, then every other row cleared in column q
            if (tid < rank) Km[q][tid] = (tid == q ? 1.0 : Km[q][tid]) / piv;
            __syncthreads();
            for (int e = tid; e < rank * rank; e += NT) {
                const int i = e / rank, j = e - i * rank;
                if (i == q) continue;
                const double f = Km[i][q];
                // column q of the other rows becomes -f / piv (the inverse's column)
                Wm[i][j] = j == q ? -f * Km[q][q] : Km[i][j] - f * Km[q][j];
            }
            __syncthreads();
            for (int e = tid; e < rank * rank; e += NT) {
                const int i = e / rank, j = e - i * rank;
                if (i != q) Km[i][j] = Wm[i][j];
            }
            __syncthreads();
        }
        for (int e = tid; e < nn * rank; e += NT) {
            const int i = e / rank, c = e - i * rank;
            double s = 0.0;
            for (int a = 0; a < rank; ++a) s += Fm[i][a] * Km[a][c];
            Wm[i][c] = s;
        }
        __syncthreads();
        for (int e = tid; e < nn * nn; e += NT) {
            const int i = e / nn, j = e - i * nn;
            double s = 0.0;
            for (int a = 0; a < rank; ++a) s += Wm[i][a] * Fm[j][a];
            Cb[e] = (float)s;
        }
    }
    if (tid == 0) flags[b] = 0;
}

// Z = X W_res in split-K parts: Zp[s][row][col] = sum over the s-th of S
// equal splits of c1 of X[row][k] W_res[k][col] (W_res^T in fragment order,
// see DecodeArgs).  Grid (c2 / 64, S, row blocks of 64).  Each wavefront
// streams a contiguous quarter of the split for all 64 columns of the block
// and every row of it: each load of W_res, and of the small X operand (in
// fragment order too, read from L2 once per 64 output columns), reads 1 KB of
// consecutive bytes.  The wavefronts' partial sums meet in LDS.  Bound by the single pass over W_res (HBM); the
// split keeps every compute unit streaming when c2 is narrow (the down
// projection).
template <typename E, bool TWO>
__global__ __launch_bounds__(NT) void decode_z_kernel(const E *__restrict__ X, const E *__restrict__ Wres_t,
                                                      int64_t N, int64_t c1, int64_t c2, int splits,
                                                      float *__restrict__ Zp) {
    __shared__ float red[2][kRowBlock * kZCols];  // two wavefronts' partials [row][col]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int64_t col0 = (int64_t)blockIdx.x * kZCols;
    const int s = blockIdx.y;
    const int64_t row0 = (int64_t)blockIdx.z * kRowBlock;
    typedef typename Frag<E>::type F;
    const int64_t c0 = col0 + lr, c1b = col0 + 32 + lr;
    const bool c0_ok = c0 < c2, c1_ok = c1b < c2;
    const int64_t ra = row0 + lr, rb = row0 + 32 + lr;
    const bool a_ok = ra < N, b_ok = rb < N;
    // W_res^T in fragment order: block (32-column block cb, 16-deep step ks)
    // at element 512 (cb c1 / 16 + ks); this lane's 8 elements at 8 lane
    const int64_t cb0 = col0 / 32, cb1 = c1_ok ? cb0 + 1 : cb0;
    const E *pb0 = Wres_t + cb0 * 32 * c1 + 8 * lane, *pb1 = Wres_t + cb1 * 32 * c1 + 8 * lane;
    // X in fragment order (left by decode_project_kernel): the block's two
    // 32-row blocks, the second clamped to the last one stored (its rows are
    // masked)
    const int64_t rblk = row0 / 32, nrb = (N + 31) / 32;
    const E *pa0 = X + rblk * 32 * c1 + 8 * lane;
    const E *pa1 = X + (rblk + 1 < nrb ? rblk + 1 : rblk) * 32 * c1 + 8 * lane;
    // this wavefront's contiguous quarter of split s (whole 16-deep steps)
    const int64_t ks = c1 / splits, kbeg = (int64_t)s * ks;
    const int64_t q4 = ((ks + 63) / 64) * 16;
    const int64_t kb = kbeg + (wave * q4 < ks ? wave * q4 : ks);
    const int64_t ke = kbeg + ((wave + 1) * q4 < ks ? (wave + 1) * q4 : ks);
    f32x16 z00 = f32x16{}, z01 = f32x16{}, z10 = f32x16{}, z11 = f32x16{};
    // two register sets: the next batch's loads are requested before the
    // current batch's MFMAs; loads are unconditional (steps past ke reread
    // kbeg) and zeroed at the MFMA
    constexpr int U = kUnrollRes;
    auto load = [&](int64_t k0, F (&b0)[U], F (&b1)[U], F (&a0)[U], F (&a1)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = k0 + 16 * u;
            const int64_t kk = k < ke ? k : kbeg;
            b0[u] = ld_frag(pb0 + 32 * kk);
            b1[u] = ld_frag(pb1 + 32 * kk);
            a0[u] = ld_frag(pa0 + 32 * kk);
            if constexpr (TWO) a1[u] = ld_frag(pa1 + 32 * kk);
        }
    };
    auto mma = [&](int64_t k0, const F (&b0)[U], const F (&b1)[U], const F (&a0)[U], const F (&a1)[U])
                   __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool kin = k0 + 16 * u < ke;
            const F x0 = keep_if(kin && a_ok, a0[u]);
            const F w0 = keep_if(c0_ok, b0[u]), w1 = keep_if(c1_ok, b1[u]);
            z00 = mma16(z00, x0, w0);
            z01 = mma16(z01, x0, w1);
            if constexpr (TWO) {
                const F x1 = keep_if(kin && b_ok, a1[u]);
                z10 = mma16(z10, x1, w0);
                z11 = mma16(z11, x1, w1);
            }
        }
    };
    {
        F sb0[U], sb1[U], sa0[U], sa1[U], tb0[U], tb1[U], ta0[U], ta1[U];
        constexpr int64_t BS = 16 * U;  // K advance of one batch
        int64_t k0 = kb;
        load(k0, sb0, sb1, sa0, sa1);
        __builtin_amdgcn_sched_barrier(0);
        for (; k0 < ke; k0 += 2 * BS) {
            load(k0 + BS, tb0, tb1, ta0, ta1);
            mma(k0, sb0, sb1, sa0, sa1);
            __builtin_amdgcn_sched_barrier(0);
            load(k0 + 2 * BS, sb0, sb1, sa0, sa1);
            mma(k0 + BS, tb0, tb1, ta0, ta1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // wavefronts 0 and 1 write their sums, 2 and 3 add theirs, then the two
    // buffers are summed on the way out
    auto put = [&](float *buf, bool add) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int r = acc_row(lane, t);
            float *p00 = buf + r * kZCols + lr, *p01 = p00 + 32;
            float *p10 = buf + (32 + r) * kZCols + lr, *p11 = p10 + 32;
            *p00 = add ? *p00 + z00[t] : z00[t];
            *p01 = add ? *p01 + z01[t] : z01[t];
            if constexpr (TWO) {
                *p10 = add ? *p10 + z10[t] : z10[t];
                *p11 = add ? *p11 + z11[t] : z11[t];
            }
        }
    };
    if (wave < 2) put(red[wave], false);
    __syncthreads();
    if (wave >= 2) put(red[wave - 2], true);
    __syncthreads();
    const int rows = TWO ? kRowBlock : 32;
    for (int e = tid; e < rows * kZCols; e += NT) {
        const int r = e / kZCols, c = e % kZCols;
        if (row0 + r < N && col0 + c < c2) Zp[((int64_t)s * N + row0 + r) * c2 + col0 + c] = red[0][e] + red[1][e];
    }
}

// Y[rows][col0..col0+32) = T_s V_s^T + bias + alpha blockdiag(C_b) Z with
// Z = X W_res summed over decode_z_kernel's splits (§2.4's fused output with
// bias and correction weight alpha).  Grid (c2/32, row blocks of whole
// instances).  Each wavefront takes a contiguous quarter of the V_s
// contraction (measured 11-15 % faster per decode step than dealing the
// 16-deep steps round-robin, whose loads touch 32 bytes of 32 lines each),
// and the quarters are reduced in LDS.
template <typename E, bool TWO>
__global__ __launch_bounds__(NT) void decode_output_kernel(const float *__restrict__ Zp, int zsplits,
                                                           const E *__restrict__ Tt,
                                                           const float *__restrict__ coef,
                                                           const E *__restrict__ Vs, int64_t N, int64_t n,
                                                           int64_t c2, int kw, int64_t rows_blk,
                                                           const E *__restrict__ bias, float alpha,
                                                           E *__restrict__ Y) {
    __shared__ float part[NT / 64][kRowBlock * 32];  // each wavefront's partial [row][col]
    __shared__ float Zs[kRowBlock][33];              // Z of the block's rows
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
    // Z of the block, summed over the splits (read before the V_s stream so
    // that its latency hides behind it)
    for (int e = tid; e < kRowBlock * 32; e += NT) {
        const int r = e >> 5, c = e & 31;
        float z = 0.f;
        if (row0 + r < row_end && col0 + c < c2)
            for (int q = 0; q < zsplits; ++q) z += Zp[((int64_t)q * N + row0 + r) * c2 + col0 + c];
        Zs[r][c] = z;
    }
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    const int64_t rac = a_ok ? ra : row0, rbc = b_ok ? rb : row0;
    {
        // V_s in fragment order: block (32-column block, 16-deep step k / 16)
        // at element 512 (col0 / 32 * kw / 16 + k / 16)
        const E *pb = Vs + (col0 / 32) * 32 * kw + 8 * lane;
        // T_s in fragment order (left by the coefficient kernel); a row block
        // of whole instances need not start on a 32-row boundary, so each
        // lane addresses its own row
        const E *pa0 = Tt + frag_index(rac, lk, kw), *pa1 = Tt + frag_index(rbc, lk, kw);
        const int q4 = ((kw + 63) / 64) * 16;
        const int vb = wave * q4 < kw ? wave * q4 : kw, ve = (wave + 1) * q4 < kw ? (wave + 1) * q4 : kw;
        for (int k0 = vb; k0 < ve; k0 += 16 * kUnroll) {
            F fb[kUnroll], fa0[kUnroll], fa1[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int k = k0 + 16 * u;
                const bool kin = k < ve;
                const int kk = kin ? k : 0;
                fb[u] = keep_if(kin && col_ok, ld_frag(pb + 32 * kk));
                fa0[u] = keep_if(kin && a_ok, ld_frag(pa0 + 32 * kk));
                if constexpr (TWO) fa1[u] = keep_if(kin && b_ok, ld_frag(pa1 + 32 * kk));
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                s0 = mma16(s0, fa0[u], fb[u]);
                if constexpr (TWO) s1 = mma16(s1, fa1[u], fb[u]);
            }
        }
    }
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

size_t decode_workspace_bytes(int64_t B, int64_t n, int64_t c1, int64_t c2, int kw, int kc) {
    return dual_layout(B, n, c1, c2, kw, kc).total;
}

template <typename E> hipError_t launch_decode_project(const DecodeArgs<E> &a, hipStream_t st) {
    const DualLayout L = dual_layout(a.B, a.n, a.c1, a.c2, a.kw, a.kc);
    const int64_t N = a.B * a.n;
    const int K1 = a.kw + a.kc;
    dim3 grid((unsigned)((K1 + 31) / 32), (unsigned)L.splits, (unsigned)((N + kRowBlock - 1) / kRowBlock));
    if (N > 32)
        hipLaunchKernelGGL((decode_project_kernel<E, true>), grid, dim3(NT), 0, st, a.X, a.Aext, N, a.c1, K1,
                           L.splits, (float *)(a.ws + L.partial), (E *)(a.ws + L.Xt));
    else
        hipLaunchKernelGGL((decode_project_kernel<E, false>), grid, dim3(NT), 0, st, a.X, a.Aext, N, a.c1, K1,
                           L.splits, (float *)(a.ws + L.partial), (E *)(a.ws + L.Xt));
    return hipGetLastError();
}

template <typename E> hipError_t launch_decode_coef(const DecodeArgs<E> &a, hipStream_t st) {
    const DualLayout L = dual_layout(a.B, a.n, a.c1, a.c2, a.kw, a.kc);
    const int64_t N = a.B * a.n;
    if (a.n > 16) {
        if (a.n > kWideTokens || a.lambda != 0.f || a.kc > kMaxCorr) return hipErrorInvalidValue;
        hipLaunchKernelGGL((decode_coef_wide_kernel<E>), dim3((unsigned)a.B), dim3(NT), 0, st,
                           (const float *)(a.ws + L.partial), N, a.n, a.kw + a.kc, a.kw, a.k_real, L.splits,
                           (float *)(a.ws + L.T), (E *)(a.ws + L.Tt), (float *)(a.ws + L.coef), a.flags);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_coef_kernel<E>), dim3((unsigned)a.B), dim3(NT), 0, st,
                       (const float *)(a.ws + L.partial), N, a.n, a.kw + a.kc, a.kw, a.k_real, L.splits, a.lambda,
                       (float *)(a.ws + L.T), (E *)(a.ws + L.Tt), (float *)(a.ws + L.coef), a.flags);
    return hipGetLastError();
}

template <typename E> hipError_t launch_decode_output(const DecodeArgs<E> &a, hipStream_t st) {
    const DualLayout L = dual_layout(a.B, a.n, a.c1, a.c2, a.kw, a.kc);
    const int64_t N = a.B * a.n;
    float *const Zp = (float *)(a.ws + L.zpart);
    // Z = X W_res by splits; the second 32-row MFMA block only when N needs it
    const dim3 zgrid((unsigned)((a.c2 + kZCols - 1) / kZCols), (unsigned)L.zsplits,
                     (unsigned)((N + kRowBlock - 1) / kRowBlock));
    if (N > 32)
        hipLaunchKernelGGL((decode_z_kernel<E, true>), zgrid, dim3(NT), 0, st, (const E *)(a.ws + L.Xt), a.Wres_t,
                           N, a.c1, a.c2, L.zsplits, Zp);
    else
        hipLaunchKernelGGL((decode_z_kernel<E, false>), zgrid, dim3(NT), 0, st, (const E *)(a.ws + L.Xt),
                           a.Wres_t, N, a.c1, a.c2, L.zsplits, Zp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rb = rows_per_block(a.n);
    dim3 grid((unsigned)((a.c2 + 31) / 32), (unsigned)((N + rb - 1) / rb));
    // the second 32-row MFMA block only when some row block has rows there
    if (std::min<int64_t>(rb, N) > 32)
        hipLaunchKernelGGL((decode_output_kernel<E, true>), grid, dim3(NT), 0, st, (const float *)Zp, L.zsplits,
                           (const E *)(a.ws + L.Tt), (const float *)(a.ws + L.coef), a.Vs, N, a.n, a.c2,
                           a.kw, rb, a.bias, a.alpha, a.Y);
    else
        hipLaunchKernelGGL((decode_output_kernel<E, false>), grid, dim3(NT), 0, st, (const float *)Zp, L.zsplits,
                           (const E *)(a.ws + L.Tt), (const float *)(a.ws + L.coef), a.Vs, N, a.n, a.c2,
                           a.kw, rb, a.bias, a.alpha, a.Y);
    return hipGetLastError();
}

template hipError_t launch_decode_project<bf16>(const DecodeArgs<bf16> &, hipStream_t);
template hipError_t launch_decode_coef<bf16>(const DecodeArgs<bf16> &, hipStream_t);
template hipError_t launch_decode_output<bf16>(const DecodeArgs<bf16> &, hipStream_t);
template hipError_t launch_decode_project<float>(const DecodeArgs<float> &, hipStream_t);
template hipError_t launch_decode_coef<float>(const DecodeArgs<float> &, hipStream_t);
template hipError_t launch_decode_output<float>(const DecodeArgs<float> &, hipStream_t);

}  // namespace dyra
