// Fused output kernel of the DyRA forward path for gfx950.
//
// "DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
// DNNs", Eq. 6 / Algorithm 1 line 13 with the static part written as in
// Proposition 1 (Eq. 8): for a tile of BM token rows
//
//     Y[rows] = T_s V_s^T + L1 R1_b,   T_s = X[rows] A_s,
//
// with T = [T_s | L1] held in LDS for the whole tile (it never goes to HBM)
// and the correction accumulated into the same registers as the static part
// before Y is stored once (the fused merge of §2.4).
//
// Phase 1 (T_s): the X tile streams through LDS in 32-deep slices; each
// wavefront owns up to four 32-column blocks of T_s and reads their A_s
// fragments straight from global memory (L2), one slice ahead.
// Phase 2 (Y): each wavefront owns 128 output features x all BM tokens and
// walks the features in steps of 512 with no barriers: A operands (rows of V_s
// and of R1_b) come from global memory two k-steps ahead, B operands (T rows)
// from LDS.  Computing the transposed block puts four consecutive features of
// one token in a lane, so Y is written in 8-byte (bf16) / 16-byte (fp32) runs.
// A tile that straddles instances runs the correction once per instance with
// the other instance's token lanes masked to zero.
#include "dyra_kernels.h"

#include <algorithm>

#include "mfma_tile.h"

namespace dyra {

namespace {

constexpr int NT = 256;

template <typename E> constexpr int out_bk() { return sizeof(E) == 2 ? 32 : 16; }

template <typename E>
__device__ __forceinline__ void store4(E *p, const float (&v)[4]) {
    if constexpr (sizeof(E) == 2) {
        union { uint2 u; bf16 e[4]; } w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w.e[q] = to_elem<E>(v[q]);
        *reinterpret_cast<uint2 *>(p) = w.u;
    } else {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

template <typename E, int BM, int NB>
__global__ __launch_bounds__(NT) void output_kernel(const E *__restrict__ X, int64_t N, int64_t n, int64_t c1,
                                                    int64_t c2, const E *__restrict__ Aext, int kw, int kc,
                                                    const E *__restrict__ Vs, const E *__restrict__ L1,
                                                    const E *__restrict__ R1t, E *__restrict__ Y) {
    constexpr int BK = out_bk<E>();
    constexpr int RB = BM / 32;   // token blocks per tile
    constexpr int FB = 4;         // output-feature blocks per wavefront in phase 2
    constexpr int VEC = Lay<E>::VEC;
    typedef typename Frag<E>::type F;
    using CX = SliceCopy<E, BM, BK, NT>;
    extern __shared__ __align__(16) char smem[];
    const int K1 = kw + kc;
    const int TS = K1 + Lay<E>::PAD;
    E *const T = reinterpret_cast<E *>(smem);
    // X staging buffers follow T: buffer s at sXb + s * BM * CX::STRIDE
    E *const sXb = T + BM * TS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    const int64_t row0 = (int64_t)blockIdx.x * BM;

    // ---------------- phase 1: T_s = X[rows] A_s
    const int nblk = kw / 32;
    for (int p0 = 0; p0 < nblk; p0 += 4 * NB) {
        f32x16 acc[RB][NB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int q = 0; q < NB; ++q) acc[i][q] = f32x16{};
        int colq[NB];
        bool okq[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int blk = p0 + wave + 4 * q;
            okq[q] = blk < nblk;
            colq[q] = blk * 32 + lr;
        }
        const int64_t S = c1 / BK;
        CX cx;
        // A_s fragments of two consecutive slices alternate between fa and fb
        F fa[BK / 16][NB], fb[BK / 16][NB];
        auto load_a = [&](F (&f)[BK / 16][NB], int64_t k0) {
#pragma unroll
            for (int s16 = 0; s16 < BK / 16; ++s16)
#pragma unroll
                for (int q = 0; q < NB; ++q)
                    f[s16][q] = okq[q] ? ld_frag(Aext + (int64_t)colq[q] * c1 + k0 + s16 * 16 + lk) : F{};
        };
        auto mma_x = [&](const F (&f)[BK / 16][NB], int64_t s) {
            const E *xs = sXb + (int)(s & 1) * (BM * CX::STRIDE) + lr * CX::STRIDE + lk;
#pragma unroll
            for (int s16 = 0; s16 < BK / 16; ++s16) {
                F fx[RB];
#pragma unroll
                for (int i = 0; i < RB; ++i) fx[i] = ld_frag(xs + i * 32 * CX::STRIDE + s16 * 16);
#pragma unroll
                for (int q = 0; q < NB; ++q)
                    if (okq[q])
#pragma unroll
                        for (int i = 0; i < RB; ++i) acc[i][q] = mma16(acc[i][q], fx[i], f[s16][q]);
            }
        };
        cx.load(X, c1, row0, N, 0, tid);
        load_a(fa, 0);
        cx.store(sXb, tid);
        __syncthreads();
        for (int64_t s = 0; s < S; s += 2) {
            // slice s with fa, slice s+1 with fb
            if (s + 1 < S) {
                cx.load(X, c1, row0, N, (s + 1) * BK, tid);
                load_a(fb, (s + 1) * BK);
            }
            mma_x(fa, s);
            if (s + 1 < S) cx.store(sXb + (int)((s + 1) & 1) * (BM * CX::STRIDE), tid);
            __syncthreads();
            if (s + 1 < S) {
                if (s + 2 < S) {
                    cx.load(X, c1, row0, N, (s + 2) * BK, tid);
                    load_a(fa, (s + 2) * BK);
                }
                mma_x(fb, s + 1);
                if (s + 2 < S) cx.store(sXb + (int)((s + 2) & 1) * (BM * CX::STRIDE), tid);
                __syncthreads();
            }
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            if (!okq[q]) continue;
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int t = 0; t < 16; ++t) T[(i * 32 + acc_row(lane, t)) * TS + colq[q]] = to_elem<E>(acc[i][q][t]);
        }
    }
    // ---------------- the tile's L1 rows next to T_s
    if (kc > 0) {
        const int lchunks = kc / VEC;
        for (int e = tid; e < BM * lchunks; e += NT) {
            const int r = e / lchunks, k0 = (e - r * lchunks) * VEC;
            const uint4 v = (row0 + r < N) ? *reinterpret_cast<const uint4 *>(L1 + (row0 + r) * kc + k0)
                                          : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(T + r * TS + kw + k0) = v;
        }
    }
    __syncthreads();

    // ---------------- phase 2: Y^T blocks [features][tokens], no barriers
    const int64_t row_end = (row0 + BM < N) ? row0 + BM : N;
    const int64_t b_first = row0 / n, b_last = (row_end - 1) / n;
    const E *tb = T + lr * TS + lk;
    for (int64_t f0 = (int64_t)wave * 32 * FB; f0 < c2; f0 += 4 * 32 * FB) {
        f32x16 acc[FB][RB];
#pragma unroll
        for (int j = 0; j < FB; ++j)
#pragma unroll
            for (int i = 0; i < RB; ++i) acc[j][i] = f32x16{};
        int64_t frow[FB];
        bool fok[FB];
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            frow[j] = f0 + j * 32 + lr;
            fok[j] = frow[j] < c2;
        }
        // static part, K = kw, in 32-deep steps with the next step's V_s rows in flight
        if (kw > 0) {
            // two 32-deep stages of V_s fragments alternate, the next one in flight
            F va[2][FB], vb[2][FB];
            auto load_v = [&](F (&v)[2][FB], int k) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < FB; ++j) v[h][j] = fok[j] ? ld_frag(Vs + frow[j] * kw + k + h * 16 + lk) : F{};
            };
            auto mma_v = [&](const F (&v)[2][FB], int k) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    F ft[RB];
#pragma unroll
                    for (int i = 0; i < RB; ++i) ft[i] = ld_frag(tb + i * 32 * TS + k + h * 16);
#pragma unroll
                    for (int j = 0; j < FB; ++j)
#pragma unroll
                        for (int i = 0; i < RB; ++i) acc[j][i] = mma16(acc[j][i], v[h][j], ft[i]);
                }
            };
            load_v(va, 0);
            for (int k = 0; k < kw; k += 64) {
                if (k + 32 < kw) load_v(vb, k + 32);
                mma_v(va, k);
                if (k + 64 < kw) load_v(va, k + 64);
                if (k + 32 < kw) mma_v(vb, k + 32);
            }
        }
        // correction, K = kc, once per instance present in the tile
        for (int64_t b = b_first; b <= b_last && kc > 0; ++b) {
            const int64_t ib0 = b * n, ib1 = ib0 + n;
            const E *rb = R1t + b * c2 * kc;
            for (int k = 0; k < kc; k += 16) {
                F fr[FB];
#pragma unroll
                for (int j = 0; j < FB; ++j) fr[j] = fok[j] ? ld_frag(rb + frow[j] * kc + k + lk) : F{};
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const int64_t blk0 = row0 + i * 32;
                    if (blk0 >= ib1 || blk0 + 32 <= ib0) continue;
                    const int64_t r = blk0 + lr;
                    F ft = ld_frag(tb + i * 32 * TS + kw + k);
                    if (!(r >= ib0 && r < ib1 && r < N)) ft = zero_frag(ft);
#pragma unroll
                    for (int j = 0; j < FB; ++j) acc[j][i] = mma16(acc[j][i], fr[j], ft);
                }
            }
        }
        // store: lane = token, 4 consecutive features per register group
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int64_t r = row0 + i * 32 + lr;
            if (r >= N) continue;
#pragma unroll
            for (int j = 0; j < FB; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t f = f0 + j * 32 + acc_row(lane, 4 * g);
                    if (f >= c2) continue;
                    const float v[4] = {acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2],
                                        acc[j][i][4 * g + 3]};
                    store4<E>(Y + r * c2 + f, v);
                }
        }
    }
}

template <typename E> size_t output_smem_bytes(int bm, int kw, int kc) {
    const size_t es = sizeof(E);
    const size_t pad = Lay<E>::PAD;
    return es * ((size_t)bm * (kw + kc + pad) + 2 * (size_t)bm * (out_bk<E>() + pad));
}

template <typename E, int BM, int NB>
hipError_t output_launch(const E *X, int64_t N, int64_t n, int64_t c1, int64_t c2, const E *Aext, int kw, int kc,
                         const E *Vs, const E *L1, const E *R1t, E *Y, hipStream_t st) {
    auto kfn = output_kernel<E, BM, NB>;
    const size_t smem = output_smem_bytes<E>(BM, kw, kc);
    hipError_t e = hipFuncSetAttribute((const void *)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kfn, dim3((unsigned)((N + BM - 1) / BM)), dim3(NT), smem, st, X, N, n, c1, c2, Aext, kw, kc, Vs,
                       L1, R1t, Y);
    return hipGetLastError();
}

}  // namespace

template <typename E>
hipError_t launch_output(const E *X, int64_t N, int64_t n, int64_t c1, int64_t c2, const E *Aext, int kw, int kc,
                         const E *Vs, const E *L1, const E *R1t, E *Y, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    // column blocks of T_s per wavefront in one pass of phase 1 (at most 4)
    const int nb = std::min(4, std::max(1, (kw / 32 + 3) / 4));
#define DYRA_OUT(BM)                                                                                              \
    switch (nb) {                                                                                                 \
    case 1: return output_launch<E, BM, 1>(X, N, n, c1, c2, Aext, kw, kc, Vs, L1, R1t, Y, st);                    \
    case 2: return output_launch<E, BM, 2>(X, N, n, c1, c2, Aext, kw, kc, Vs, L1, R1t, Y, st);                    \
    case 3: return output_launch<E, BM, 3>(X, N, n, c1, c2, Aext, kw, kc, Vs, L1, R1t, Y, st);                    \
    default: return output_launch<E, BM, 4>(X, N, n, c1, c2, Aext, kw, kc, Vs, L1, R1t, Y, st);                   \
    }
    if (output_smem_bytes<E>(128, kw, kc) <= kMaxLds) { DYRA_OUT(128) }
    if (output_smem_bytes<E>(64, kw, kc) <= kMaxLds) { DYRA_OUT(64) }
    if (output_smem_bytes<E>(32, kw, kc) <= kMaxLds) { DYRA_OUT(32) }
#undef DYRA_OUT
    return hipErrorInvalidValue;
}

bool output_fits(size_t elem_bytes, int kw, int kc) {
    return elem_bytes == 2 ? output_smem_bytes<bf16>(32, kw, kc) <= kMaxLds
                           : output_smem_bytes<float>(32, kw, kc) <= kMaxLds;
}

template hipError_t launch_output<bf16>(const bf16 *, int64_t, int64_t, int64_t, int64_t, const bf16 *, int, int,
                                        const bf16 *, const bf16 *, const bf16 *, bf16 *, hipStream_t);
template hipError_t launch_output<float>(const float *, int64_t, int64_t, int64_t, int64_t, const float *, int, int,
                                         const float *, const float *, const float *, float *, hipStream_t);

}  // namespace dyra
