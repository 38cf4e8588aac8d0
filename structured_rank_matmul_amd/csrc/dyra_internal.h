// Internal declarations shared by the host factorisation and the HIP library.
#pragma once

#include <cstdint>
#include <vector>

#include "../../include/dyra.h"

namespace dyra {

// Float64 factors of one layer (Algorithm 1, Offline Preparation).
struct Factors {
    int64_t c1 = 0, c2 = 0;
    int32_t r = 0, k = 0;
    double lambda = 0.0;
    std::vector<double> A_s;    // [c1][r]   U_r Sigma_r
    std::vector<double> V_s;    // [c2][r]   V_r
    std::vector<double> R0;     // [k][c2]   fixed initial right factor
    std::vector<double> P_L;    // [c1][k]   W_res R0^T (R0 R0^T + lambda I)^-1
    std::vector<double> sigma;  // [r + k]   leading singular values
    std::vector<double> W_res;  // [c1][c2]  W - A_s V_s^T
};

// R0_in: host float32 [k][c2] to use as R^(0) (e.g. a Gaussian draw, §2.2
// Fig. 2), or null for the top-k right singular vectors of W_res (Appendix D).
dyra_status factorize(const float *W, int64_t c1, int64_t c2, int32_t r, int32_t k, double lambda,
                      Factors *out, const float *R0_in = nullptr);

// Preparation with a BLAST W_hat (Appendix B) from the caller's factors:
// U [c1][rb] (block row i = rows i*c1/nb ..), S [nb][nb][rb] (diagonal
// couplings s_ij), V [c2][rb]; all float32 host arrays.  Fills W_res, R0 and
// P_L (A_s, V_s and sigma stay empty).
dyra_status factorize_blast(const float *W, int64_t c1, int64_t c2, int32_t nb, int32_t rb, const float *U,
                            const float *S, const float *V, int32_t k, double lambda, Factors *out);

}  // namespace dyra
