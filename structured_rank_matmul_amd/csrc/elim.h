// Lane-per-row elimination of a small SPD matrix in one wavefront (gfx950),
// shared by the SPD solves of the DyRA correction (solve.hip, als.hip).
//
// Lane i holds row i of the k x k matrix G in g[0..k) and one further row of
// right-hand data in l[0..k).  Step K takes pivot row K (lane K) to every
// lane through v_readlane, so the factorisation needs no barrier and no LDS.
// After elim_step<KC, 0>:
//   g[0..i] of lane i is row i of the Cholesky factor C (G = C C^T); entries
//     past the diagonal are left over and meaningless;
//   l of every lane is l C^-T (the row solved against C^T).
// back_step<KC, KC - 1> then turns a row u (as left in l) into u C^-1.
#pragma once

#include <hip/hip_runtime.h>

namespace dyra {

__device__ __forceinline__ float bcast(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// One elimination step (step K, pivot row K held by lane K).  Lane i holds
// row i of the trailing matrix in g and its data row in l.  The pivot row's
// entries are broadcast to SGPRs in batches of 8 ahead of the FMAs that use
// them.
template <int KC, int K, int M0>
__device__ __forceinline__ void elim_batch(float (&g)[KC], float (&l)[KC], float a, float bt) {
    constexpr int CNT = (KC - M0) < 8 ? (KC - M0) : 8;
    float sv[CNT];
#pragma unroll
    for (int u = 0; u < CNT; ++u) sv[u] = bcast(g[M0 + u], K);  // trailing row K = C[m][K] C[K][K]
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CNT; ++u) {
        g[M0 + u] = fmaf(-a, sv[u], g[M0 + u]);
        l[M0 + u] = fmaf(-bt, sv[u], l[M0 + u]);
    }
    // the batch's FMAs complete here, so its broadcasts die here (otherwise
    // the compiler may defer the token-row FMAs and spill the SGPRs)
#pragma unroll
    for (int u = 0; u < CNT; ++u) asm volatile("" : "+v"(g[M0 + u]), "+v"(l[M0 + u]));
    if constexpr (M0 + 8 < KC) elim_batch<KC, K, M0 + 8>(g, l, a, bt);
}

template <int KC, int K>
__device__ __forceinline__ void elim_step(float (&g)[KC], float (&l)[KC], int kc_real, float th, bool &fail) {
    if constexpr (K < KC) {
        float pk = bcast(g[K], K);
        const bool bad = K < kc_real && !(pk > th);  // padding pivots are 1
        fail = fail || bad;
        pk = bad ? 1.f : pk;
        const float rp = __builtin_amdgcn_rcpf(pk);
        const float rs = __builtin_amdgcn_rsqf(pk);
        const float a = g[K] * rp;   // G rows: C[i][K] / C[K][K]
        const float bt = l[K] * rp;  // token rows: Q[t][K] / C[K][K]
        l[K] = l[K] * rs;
        g[K] = g[K] * rs;            // C[i][K]; column K of g is not read again
        if constexpr (K + 1 < KC) elim_batch<KC, K, K + 1>(g, l, a, bt);
        elim_step<KC, K + 1>(g, l, kc_real, th, fail);
    }
}

// Back substitution x C = u for lower-triangular C whose row j sits in g of
// lane j (as elim_step leaves it): column J from the last down, x_J = u_J /
// C[J][J], then u_m -= x_J C[J][m] for m < J, the C[J][m] broadcast in batches
// of 8 as in elim_batch.  u becomes x.
template <int KC, int J, int M0>
__device__ __forceinline__ void back_batch(const float (&g)[KC], float (&u)[KC], float x) {
    constexpr int CNT = (J - M0) < 8 ? (J - M0) : 8;
    float sv[CNT];
#pragma unroll
    for (int q = 0; q < CNT; ++q) sv[q] = bcast(g[M0 + q], J);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < CNT; ++q) u[M0 + q] = fmaf(-x, sv[q], u[M0 + q]);
#pragma unroll
    for (int q = 0; q < CNT; ++q) asm volatile("" : "+v"(u[M0 + q]));
    if constexpr (M0 + 8 < J) back_batch<KC, J, M0 + 8>(g, u, x);
}

template <int KC, int J>
__device__ __forceinline__ void back_step(const float (&g)[KC], float (&u)[KC]) {
    if constexpr (J >= 0) {
        const float x = u[J] * __builtin_amdgcn_rcpf(bcast(g[J], J));
        u[J] = x;
        if constexpr (J > 0) back_batch<KC, J, 0>(g, u, x);
        back_step<KC, J - 1>(g, u);
    }
}

}  // namespace dyra
