// Tiled MFMA GEMM for gfx950: D = A B^T with both operands K-contiguous.
//
// Used for the exact product X W (the dense reference, §2.1 Eq. 2), the left
// factor L1 = X P_L (DyRA paper Eq. 7) and the stacked right factor
// R1 = M' W_res of all instances at once (Eq. 5; the O(c1 c2 r) term of §2.3).
//
// A workgroup owns a BM x BN output tile and four wavefronts each own a
// (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks.  K advances in slices of 64
// (bf16) or 32 (fp32) elements staged through two LDS buffers: the next slice
// is fetched into registers while the current one feeds the MFMAs.  Tiles are
// handed out XCD by XCD: workgroup ids are dealt round-robin over the 8 XCDs,
// so id i works on tile (i % 8) * ceil(T/8) + i / 8 and each XCD's L2 sees a
// contiguous band of tiles that share operand panels.
#include "dyra_kernels.h"

#include <cmath>

#include "mfma_tile.h"

namespace dyra {

namespace {

template <typename E> constexpr int gemm_bk() { return sizeof(E) == 2 ? 64 : 32; }

// Four consecutive values of one row of a row-major D (columns j..j+3).
template <typename E> struct RowStore {
    E *D;
    int64_t ldd;
    __device__ __forceinline__ void operator()(int64_t i, int64_t j, const float (&v)[4]) const {
        E *p = D + i * ldd + j;
        if constexpr (sizeof(E) == 2) {
            union { uint2 u; bf16 e[4]; } w;
#pragma unroll
            for (int q = 0; q < 4; ++q) w.e[q] = to_elem<E>(v[q]);
            *reinterpret_cast<uint2 *>(p) = w.u;
        } else {
            *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
};

// Four consecutive rows r..r+3 (= correction indices kk..kk+3 of instance b) of
// one column c of the stacked right factor, stored as R1t[b][c][kk..kk+3].
template <typename E> struct R1tStore {
    E *R1t;
    int64_t kc, c2;
    __device__ __forceinline__ void operator()(int64_t r, int64_t c, const float (&v)[4]) const {
        // rows are below 2^31 (instances x correction rank): 32-bit division
        const uint32_t ru = (uint32_t)r, kcu = (uint32_t)kc;
        const int64_t b = ru / kcu, kk = ru - (uint32_t)b * kcu;
        E *p = R1t + (b * c2 + c) * kc + kk;
        if constexpr (sizeof(E) == 2) {
            union { uint2 u; bf16 e[4]; } w;
#pragma unroll
            for (int q = 0; q < 4; ++q) w.e[q] = to_elem<E>(v[q]);
            *reinterpret_cast<uint2 *>(p) = w.u;
        } else {
            *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
};

// ROWS = true: the epilogue receives four consecutive columns of one row (the
// MFMA is issued with the operands swapped, so a lane holds a row of the
// block); ROWS = false: four consecutive rows of one column.
template <typename E, int BM, int BN, int WM, int WN, bool ROWS, class Epi>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const E *__restrict__ A, int64_t lda, const E *__restrict__ B,
                                                  int64_t ldb, int64_t M, int64_t N, int64_t K, int tiles_n,
                                                  int ntiles, int per_xcd, Epi epi) {
    constexpr int BK = gemm_bk<E>();
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    using CA = SliceCopy<E, BM, BK, NT>;
    using CB = SliceCopy<E, BN, BK, NT>;
    extern __shared__ __align__(16) char smem[];
    // stage st holds A at lds + st * STAGE and B right after it (offsets, not a
    // pointer table, so every access stays an LDS access)
    constexpr int STAGE = BM * CA::STRIDE + BN * CB::STRIDE;
    E *const lds = reinterpret_cast<E *>(smem);
    const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (tile >= ntiles) return;
    const int64_t row0 = (int64_t)(tile / tiles_n) * BM;
    const int64_t col0 = (int64_t)(tile % tiles_n) * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
    CA ca;
    CB cb;
    // the last slice may be partial: K is a multiple of 32 (bf16) / 16 (fp32)
    const int64_t S = (K + BK - 1) / BK;
    if (S > 0) {
        ca.load(A, lda, row0, M, 0, tid, K);
        cb.load(B, ldb, col0, N, 0, tid, K);
        ca.store(lds, tid);
        cb.store(lds + BM * CA::STRIDE, tid);
    }
    __syncthreads();
    for (int64_t s = 0; s < S; ++s) {
        const int buf = (int)(s & 1);
        if (s + 1 < S) {
            ca.load(A, lda, row0, M, (s + 1) * BK, tid, K);
            cb.load(B, ldb, col0, N, (s + 1) * BK, tid, K);
        }
        const E *a = lds + buf * STAGE + (wm * TM * 32 + lr) * CA::STRIDE + lk;
        const E *b = lds + buf * STAGE + BM * CA::STRIDE + (wn * TN * 32 + lr) * CB::STRIDE + lk;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            typename Frag<E>::type fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = ld_frag(a + i * 32 * CA::STRIDE + kk);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = ld_frag(b + j * 32 * CB::STRIDE + kk);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = ROWS ? mma16(acc[i][j], fb[j], fa[i]) : mma16(acc[i][j], fa[i], fb[j]);
        }
        if (s + 1 < S) {
            ca.store(lds + (buf ^ 1) * STAGE, tid);
            cb.store(lds + (buf ^ 1) * STAGE + BM * CA::STRIDE, tid);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                const int64_t rb = row0 + wm * TM * 32 + i * 32, cb0 = col0 + wn * TN * 32 + j * 32;
                if (ROWS) {
                    const int64_t r = rb + lr, c = cb0 + acc_row(lane, 4 * g);
                    if (r < M && c < N) epi(r, c, v);
                } else {
                    const int64_t r = rb + acc_row(lane, 4 * g), c = cb0 + lr;
                    if (r < M && c < N) epi(r, c, v);
                }
            }
}

template <typename E, int BM, int BN> size_t gemm_smem() {
    constexpr int BK = gemm_bk<E>();
    return sizeof(E) * (size_t)2 * (BM + BN) * (BK + Lay<E>::PAD);
}

template <typename E, int BM, int BN, int WM, int WN, bool ROWS, class Epi>
hipError_t gemm_launch(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N, int64_t K, Epi epi,
                       hipStream_t st) {
    auto kfn = gemm_kernel<E, BM, BN, WM, WN, ROWS, Epi>;
    const size_t smem = gemm_smem<E, BM, BN>();
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int ntiles = tiles_m * tiles_n;
    const int per_xcd = (ntiles + 7) / 8;
    hipLaunchKernelGGL(kfn, dim3((unsigned)(8 * per_xcd)), dim3(64 * WM * WN), smem, st, A, lda, B, ldb, M, N, K, tiles_n,
                       ntiles, per_xcd, epi);
    return hipGetLastError();
}

// Tile shape with the smallest estimated time: rounds of 256 concurrent tiles
// times tile area, with smaller wavefront tiles charged for their higher LDS
// traffic per MFMA.
enum class Shape { T256x256, T256x128, T128x128, T64x64 };

Shape pick_shape(int64_t M, int64_t N) {
    if (N <= 64) return Shape::T64x64;
    struct C { Shape s; int bm, bn; double w; } cands[] = {
        {Shape::T256x256, 256, 256, 1.0}, {Shape::T256x128, 256, 128, 1.1}, {Shape::T128x128, 128, 128, 1.3}};
    Shape best = Shape::T128x128;
    double best_cost = 1e300;
    for (const C &c : cands) {
        const double tiles = (double)((M + c.bm - 1) / c.bm) * (double)((N + c.bn - 1) / c.bn);
        const double rounds = std::ceil(tiles / 256.0);
        const double cost = rounds * c.bm * c.bn * c.w;
        if (cost < best_cost) {
            best_cost = cost;
            best = c.s;
        }
    }
    return best;
}

template <typename E, bool ROWS, class Epi>
hipError_t gemm_dispatch(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N, int64_t K, Epi epi,
                         hipStream_t st) {
    switch (pick_shape(M, N)) {
    case Shape::T256x256: return gemm_launch<E, 256, 256, 2, 2, ROWS>(A, lda, B, ldb, M, N, K, epi, st);
    case Shape::T256x128: return gemm_launch<E, 256, 128, 2, 2, ROWS>(A, lda, B, ldb, M, N, K, epi, st);
    case Shape::T128x128: return gemm_launch<E, 128, 128, 2, 2, ROWS>(A, lda, B, ldb, M, N, K, epi, st);
    case Shape::T64x64: return gemm_launch<E, 64, 64, 2, 2, ROWS>(A, lda, B, ldb, M, N, K, epi, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

template <typename E>
hipError_t launch_gemm_store(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                             E *D, int64_t ldd, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    return gemm_dispatch<E, true>(A, lda, B, ldb, M, N, K, RowStore<E>{D, ldd}, st);
}

template <typename E>
hipError_t launch_right(const E *Mp, const E *Wres_t, int64_t rows, int64_t c1, int64_t c2, int kc, E *R1t,
                        hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    return gemm_dispatch<E, false>(Mp, c1, Wres_t, c1, rows, c2, c1, R1tStore<E>{R1t, kc, c2}, st);
}

template hipError_t launch_gemm_store<bf16>(const bf16 *, int64_t, const bf16 *, int64_t, int64_t, int64_t, int64_t,
                                            bf16 *, int64_t, hipStream_t);
template hipError_t launch_gemm_store<float>(const float *, int64_t, const float *, int64_t, int64_t, int64_t,
                                             int64_t, float *, int64_t, hipStream_t);
template hipError_t launch_right<bf16>(const bf16 *, const bf16 *, int64_t, int64_t, int64_t, int, bf16 *,
                                       hipStream_t);
template hipError_t launch_right<float>(const float *, const float *, int64_t, int64_t, int64_t, int, float *,
                                        hipStream_t);

}  // namespace dyra
