// BLAST static product, middle step (Appendix B of "DyRA: Dynamic Residual
// Approximation for Efficient Matrix Multiplication in DNNs").
//
// With W_hat's block (i, j) = U_i diag(s_ij) V_j^T, the static output of block
// column j is sum_i X_i U_i diag(s_ij) V_j^T.  The forward computes it in
// three steps: Z_i = X_i U_i (one grouped GEMM launch over the block rows),
// H_j = sum_i Z_i diag(s_ij) (this kernel), Y_j = H_j V_j^T (one grouped
// launch over the block columns, with the correction slices).  This kernel is
// elementwise across the rank index: for each token row and rank column c the nb values Z_i[c] are mixed by the
// nb x nb matrix s_..[c] into the nb values H_j[c], so it runs in place over
// T's first nb * rbp columns, and each thread owns its positions alone.
// Smix rows are rbp floats, rbp a multiple of 32, so the float4 loads and the
// LDS image stay aligned.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "dyra_kernels.h"
#include "mfma_tile.h"

namespace dyra {
namespace {

constexpr int kMixThreads = 256;
constexpr int kMixBlocks = 1024;  // four per CU: each walks several rows per thread

// Each thread owns one 16-byte chunk (VEC rank columns) of every block for a
// row and walks rows.  The couplings sit in LDS, loaded once per workgroup
// (held in registers instead, they cost every thread its own 512-byte read
// from L2 and three quarters of the register file).
template <typename E, int NB>
__global__ __launch_bounds__(kMixThreads) void blast_mix_kernel(E *__restrict__ T, int64_t ldt, int64_t N,
                                                                int rbp, const float *__restrict__ Smix) {
    constexpr int VEC = 16 / (int)sizeof(E);
    extern __shared__ __align__(16) float ss[];  // [NB][NB][rbp]
    const int t = (int)threadIdx.x;
    for (int e = 4 * t; e < NB * NB * rbp; e += 4 * kMixThreads)
        *reinterpret_cast<f32x4 *>(ss + e) = *reinterpret_cast<const f32x4 *>(Smix + e);
    __syncthreads();
    const int cpr = rbp / VEC;  // chunks per row and block
    const int rows_per_iter = kMixThreads / cpr;
    if (t >= rows_per_iter * cpr) return;
    const int c0 = (t % cpr) * VEC;
    const int64_t step = (int64_t)gridDim.x * rows_per_iter;
    for (int64_t row = (int64_t)blockIdx.x * rows_per_iter + t / cpr; row < N; row += step) {
        // keeps the coupling reads in the loop: hoisted, they take the registers back
        asm volatile("" ::: "memory");
        E *base = T + row * ldt + c0;
        u32x4 raw[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) raw[i] = *reinterpret_cast<const u32x4 *>(base + (int64_t)i * rbp);
        float z[NB][VEC];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const E *e = reinterpret_cast<const E *>(&raw[i]);
#pragma unroll
            for (int v = 0; v < VEC; ++v) z[i][v] = to_f32(e[v]);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            float h[VEC] = {};
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const float *sij = ss + (i * NB + j) * rbp + c0;
#pragma unroll
                for (int v4 = 0; v4 < VEC; v4 += 4) {
                    const f32x4 sv = *reinterpret_cast<const f32x4 *>(sij + v4);
#pragma unroll
                    for (int v = 0; v < 4; ++v) h[v4 + v] = fmaf(z[i][v4 + v], sv[v], h[v4 + v]);
                }
            }
            u32x4 out;
            E *o = reinterpret_cast<E *>(&out);
#pragma unroll
            for (int v = 0; v < VEC; ++v) o[v] = to_elem<E>(h[v]);
            *reinterpret_cast<u32x4 *>(base + (int64_t)j * rbp) = out;
        }
    }
}

// One-time set-up of a mix instantiation on the current device (its dynamic
// LDS limit: up to 128 KB at four blocks and rank 2048), under a lock.
template <typename E, int NB> hipError_t mix_setup() {
    static std::mutex mu;
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    std::lock_guard<std::mutex> lock(mu);
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute((const void *)blast_mix_kernel<E, NB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(sizeof(float) * NB * NB * 2048));
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_release);
    return hipSuccess;
}

template <typename E, int NB>
hipError_t mix_launch(E *T, int64_t ldt, int64_t N, int rbp, const float *Smix, hipStream_t st) {
    constexpr int VEC = 16 / (int)sizeof(E);
    const int rows_per_iter = kMixThreads / (rbp / VEC);
    const int64_t want = (N + rows_per_iter - 1) / rows_per_iter;
    const unsigned grid = (unsigned)(want < kMixBlocks ? want : kMixBlocks);
    const size_t smem = sizeof(float) * NB * NB * (size_t)rbp;
    const hipError_t e = mix_setup<E, NB>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((blast_mix_kernel<E, NB>), dim3(grid), dim3(kMixThreads), smem, st, T, ldt, N, rbp, Smix);
    return hipGetLastError();
}

}  // namespace

template <typename E>
hipError_t launch_blast_mix(E *T, int64_t ldt, int64_t N, int nb, int rbp, const float *Smix, hipStream_t st) {
    constexpr int VEC = 16 / (int)sizeof(E);
    if (N <= 0) return hipSuccess;
    if (rbp <= 0 || rbp % 32 != 0 || rbp / VEC > kMixThreads || ldt < (int64_t)nb * rbp || ldt % VEC != 0)
        return hipErrorInvalidValue;
    switch (nb) {
    case 1: return mix_launch<E, 1>(T, ldt, N, rbp, Smix, st);
    case 2: return mix_launch<E, 2>(T, ldt, N, rbp, Smix, st);
    case 3: return mix_launch<E, 3>(T, ldt, N, rbp, Smix, st);
    case 4: return mix_launch<E, 4>(T, ldt, N, rbp, Smix, st);
    }
    return hipErrorInvalidValue;
}

template <typename E> hipError_t blast_prepare() {
    hipError_t e;
    if ((e = mix_setup<E, 1>()) != hipSuccess) return e;
    if ((e = mix_setup<E, 2>()) != hipSuccess) return e;
    if ((e = mix_setup<E, 3>()) != hipSuccess) return e;
    return mix_setup<E, 4>();
}

template hipError_t blast_prepare<bf16>();
template hipError_t blast_prepare<float>();
template hipError_t launch_blast_mix<bf16>(bf16 *, int64_t, int64_t, int, int, const float *, hipStream_t);
template hipError_t launch_blast_mix<float>(float *, int64_t, int64_t, int, int, const float *, hipStream_t);

}  // namespace dyra
