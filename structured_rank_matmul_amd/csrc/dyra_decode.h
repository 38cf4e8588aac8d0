// Fewer tokens per instance than the correction rank (decode): the dual form.
//
// With n < k the Gram matrix L1^T L1 of Algorithm 1 line 12 is singular at
// lambda = 0, but the product L1 R1 is not: by the push-through identity
//   L1 (L1^T L1 + lambda I_k)^-1 L1^T = L1 L1^T (L1 L1^T + lambda I_n)^-1,
// so  Y_b = X_b A_s V_s^T + C_b (X_b W_res)  with the n x n matrix
//   C_b = L1_b L1_b^T (L1_b L1_b^T + lambda I_n)^-1,
// whose lambda -> 0 limit is the orthogonal projector onto the range of L1_b
// (the minimum-norm least-squares solution of Eq. 5).  For n = 1 this is the
// scalar ||l||^2 / (lambda + ||l||^2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dyra {

template <typename E> struct DecodeArgs {
    const E *X;
    int64_t B, n, c1, c2;
    int kw, kc, k_real;
    float lambda;
    const E *Aext;    // [kw + kc][c1] in MFMA fragment order, rows padded with zeros to a multiple of 32
    const E *Vs;      // [c2][kw] V_s in MFMA fragment order (512-element blocks of 32 rows x 16 deep)
    const E *Wres_t;  // [c2][c1] W_res^T in the same order
    E *Y;             // [B*n][c2]
    char *ws;         // dual-form workspace (decode_workspace_bytes)
    int *flags;       // [B]
    const E *bias;    // [c2] or null, added to every row
    float alpha;      // weight of the correction term (1 in Eq. 6)
};

size_t decode_workspace_bytes(int64_t B, int64_t n, int64_t c1, int64_t c2, int kw, int kc);

// T = X [A_s | P_L]^T as float32 partial sums over splits of c1.
template <typename E> hipError_t launch_decode_project(const DecodeArgs<E> &a, hipStream_t st);
// Sums the partials into T and forms C_b per instance.
template <typename E> hipError_t launch_decode_coef(const DecodeArgs<E> &a, hipStream_t st);
// Y = T_s V_s^T + bias + alpha blockdiag(C_b) (X W_res), streaming W_res and V_s once:
// X W_res in split-K parts first (decode_z_kernel), then the rest in one pass.
template <typename E> hipError_t launch_decode_output(const DecodeArgs<E> &a, hipStream_t st);

}  // namespace dyra
