// Lane-group helpers shared by the substitution and Newton-Schulz kernels
// (solve.hip, ns.hip): broadcast inside groups of 2 or 4 lanes by DPP, and a
// compile-time loop.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

namespace dyra {

// Broadcast within groups of G lanes (G = 1, 2 or 4) of lane q of the group,
// by DPP quad_perm (one VALU instruction, no LDS).  q is a constant once the
// caller's loop is unrolled, so the switch folds away.
template <int G> __device__ __forceinline__ float group_bcast(float v, int q) {
    if constexpr (G == 1) {
        return v;
    } else {
        int ctrl;
        if constexpr (G == 4) ctrl = q * 0x55;                                          // [q, q, q, q]
        else ctrl = q | (q << 2) | ((2 + q) << 4) | ((2 + q) << 6);                    // [q, q, 2+q, 2+q]
        const int iv = __float_as_int(v);
        int r;
        switch (ctrl) {
#define DYRA_DPP(C) case C: r = __builtin_amdgcn_mov_dpp(iv, C, 0xf, 0xf, false); break;
            DYRA_DPP(0x00) DYRA_DPP(0x55) DYRA_DPP(0xaa) DYRA_DPP(0xff) DYRA_DPP(0xa0) DYRA_DPP(0xf5)
#undef DYRA_DPP
        default: r = iv;
        }
        return __int_as_float(r);
    }
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, each i a
// compile-time constant.
template <class F, int... Is>
__device__ __forceinline__ void unroll_seq_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void unroll_seq(F &&f) {
    unroll_seq_impl(f, std::make_integer_sequence<int, N>{});
}

// Lanes per token row of the per-token substitution kernels: each lane's
// share of a k-column row must be whole 16-byte (8-column) chunks.
template <int KC> constexpr int token_lanes() { return KC % 32 == 0 ? 4 : 2; }
// Rows of a k x k factor staged in LDS at a time: the largest whole fraction
// of KC that fits in 64 KB.
template <int KC> constexpr int stage_rows() {
    int d = 1;
    while (KC % d != 0 || (KC / d) * KC * 4 > 65536) ++d;
    return KC / d;
}

}  // namespace dyra
