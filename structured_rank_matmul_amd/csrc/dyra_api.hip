// libdyra C ABI: plan preparation, workspace layout and the forward path.
//
// "DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
// DNNs", Algorithm 1 (Offline Preparation and Inference).  The host part of
// the preparation lives in host_factorize.cpp; this file rounds and packs the
// factors for the kernels, and sequences the kernels of one forward call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "dyra_internal.h"
#include "dyra_kernels.h"
#include "dyra_decode.h"

struct dyra_plan {
    int device;
    dyra_dtype dtype;
    int64_t c1, c2;
    int32_t r, k;     // static and correction ranks as requested
    int32_t kw, kc;   // padded: kw = r rounded up to 32, kc = k rounded up to 16
    float lambda;
    int32_t half_steps;  // single ALS updates: 2 = Algorithm 1 (t = 1), 3 = t 1.5, 4 = t 2, ...
    int32_t ns_iters;    // 0: Cholesky SPD solve; > 0: that many Newton-Schulz steps (§2.4)
    void *Aext;       // [kw + kc][c1]: rows 0..r-1 = A_s columns, rows kw..kw+k-1 = P_L columns
    void *Vs;         // [c2][kw]: V_s
    void *Wres_t;     // [c2][c1]: W_res transposed
    void *Wres;       // [c1][c2]: W_res (only with half_steps > 2, for the L updates)
    // The dual form's streamed operands in MFMA fragment order (frag_tile):
    // W_res^T and V_s (only for correction ranks above 0 and no BLAST W_hat)
    void *Wdec;       // tiled [c2][c1]
    void *Vdec;       // tiled [c2][kw]
    void *Adec;       // tiled Aext, rows padded with zeros to a multiple of 32
    // BLAST W_hat (Appendix B), nb > 0: kw = nb * rbp, Aext holds P_L alone
    // ([kc][c1]) and Vs is V [c2][rbp]
    int32_t nb;       // blocks per side (0: truncated-SVD W_hat)
    int32_t rbp;      // BLAST rank rounded up to 32
    void *Ublk;       // [nb * rbp][c1 / nb]: row i * rbp + c = column c of U_i
    void *Smix;       // float32 [nb][nb][rbp]: the couplings s_ij
};

// Device-side scratch of dyra_forward_noalloc: one copy per GPU, held until
// the process ends.  In host code this name is only a stand-in for the symbol;
// the device address comes from hipGetSymbolAddress (scratch_ptr below).
constexpr size_t kNoallocScratchBytes = size_t{128} << 20;
__device__ __align__(256) static char scratch[kNoallocScratchBytes];

namespace {

using dyra::bf16;

// Per-device address of `scratch`, looked up once per device with that device
// current (each GPU holds its own copy of the array at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

dyra_status scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return DYRA_ERR_NODEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device]) return DYRA_OK;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DYRA_ERR_HIP;
    g_scratch_ptr[device] = ptr;
    return DYRA_OK;
}

void *scratch_ptr(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

constexpr size_t kAlign = 256;
constexpr int kMaxCorrection = 256;
// The float32 path's SPD solve, further ALS steps and the Newton-Schulz solve
// are built for correction ranks up to 64.
constexpr int kMaxCorrectionSmall = 64;
constexpr int kMaxDualTokens = 16;       // every instance this short takes the dual form
constexpr int kMaxWideDualTokens = 64;   // the dual form for n < k at lambda = 0
constexpr int kMaxHalfSteps = 8;
constexpr int kMaxNsIters = 64;
constexpr int kMaxBlastBlocks = 4;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

size_t elem_size(dyra_dtype t) { return t == DYRA_BF16 ? 2 : 4; }

// float64 -> bfloat16 bits, round to nearest even on the float64 value.
uint16_t bf16_bits(double x) {
    float f = (float)x;  // RNE to 24 bits
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)(u >> 16);  // inf / nan
    const uint32_t low = u & 0xffffu;
    if (low == 0x8000u && (double)f != x) {
        // f sits exactly halfway between two bf16 values but x does not: the
        // float rounding decided the side, so follow x's position relative to f.
        const bool up = std::fabs(x) > std::fabs((double)f);
        return (uint16_t)((u >> 16) + (up ? 1u : 0u));
    }
    const uint32_t bias = 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)((u + bias) >> 16);
}

enum class Path { Primal, Dual, Static };

// Instances with at most kMaxDualTokens tokens take the n x n dual form: its
// eigen-decomposition stays accurate where the k x k normal equations of the
// primal form would be ill-conditioned (n close to k).  Longer instances with
// fewer tokens than the correction rank take the primal form when lambda > 0
// (the ridge keeps L1^T L1 + lambda I positive definite) and the dual form,
// with a rank-revealing factorisation, at lambda = 0 (up to
// kMaxWideDualTokens tokens).
Path path_for(const dyra_plan *p, int64_t n) {
    if (p->kc == 0) return Path::Static;
    if (p->nb > 0) return Path::Primal;  // BLAST plans have no dual form
    if (n <= kMaxDualTokens) return Path::Dual;
    if (n < p->k) return p->lambda > 0.f ? Path::Primal : Path::Dual;
    return Path::Primal;
}

// Workspace of one forward call (offsets in bytes, each 256-byte aligned):
//   flags  int32 [B]             per-instance solve failure flags
//   T      [N][kw + kc]          X A_s next to L1 (then Q) for every token
//   Qt     [B][kc][npad]         Q_b^T, token-contiguous, npad = n rounded up to 32
//                                (float32 only; bf16 reads Q_b from T)
//   Ct     float32 [B][kc][kc]   Cholesky factor of G_b by columns (bf16 only)
//   Gw     float32 [B][kp][kp]   G_b while it is factored, kp = kc rounded up to 32
//                                (bf16 with kc above 128 only; smaller G stay in LDS)
//   Mp     [B * kc][c1]          M'_b = Q_b^T X_b stacked over instances
//   R1t    [B][c2][kc]           R1_b transposed
//   with further ALS steps (half_steps > 2, als.hip):
//   C      float64 [B][kc][kc]   Cholesky factors of the last R update
//   R1row  [B*kc][c2]            R' by rows
//   Sp     [B*kc][c1]            S'^T = R' W_res^T
//   H      float32 [8][B][kc][kc] partial sums of R' R'^T
//   Kp     float32 [B][kc][kc]   the L update's coefficients
//   with the Newton-Schulz solve (ns_iters > 0):
//   F      float32               G^-1/2 per instance [B][kc][kc] (kc <= 64), or the
//                                iterates of the batched solve (ns_workspace_floats)
//   dual   decode workspace      (n <= 16 or n < k only)
struct Layout {
    size_t flags, T, Qt, Ct, Gw, Mp, R1t, C, R1row, Sp, H, Kp, F, dual, total;
    int64_t npad;
};

Layout workspace_layout(const dyra_plan *p, int64_t B, int64_t n) {
    Layout L{};
    const size_t es = elem_size(p->dtype);
    const int64_t N = B * n;
    size_t off = 0;
    L.flags = off;
    off += align_up(sizeof(int32_t) * (size_t)std::max<int64_t>(B, 1));
    if (path_for(p, n) != Path::Dual) {
        L.T = off;
        off += align_up(es * N * (p->kw + p->kc));
    }
    if (path_for(p, n) == Path::Primal) {
        L.npad = round_up(n, 32);
        L.Qt = off;
        if (p->dtype == DYRA_F32) off += align_up(es * B * p->kc * L.npad);
        L.Ct = off;
        if (p->dtype == DYRA_BF16 && p->ns_iters == 0) off += align_up(sizeof(float) * (size_t)B * p->kc * p->kc);
        L.Gw = off;
        if (p->dtype == DYRA_BF16 && p->ns_iters == 0)
            off += align_up(sizeof(float) * (size_t)B * dyra::gram_workspace_floats(p->kc));
        L.Mp = off;
        off += align_up(es * B * p->kc * p->c1);
        L.R1t = off;
        off += align_up(es * B * p->c2 * p->kc);
        if (p->ns_iters > 0) {
            L.F = off;
            off += align_up(sizeof(float) * dyra::ns_workspace_floats(B, p->kc));
        }
        if (p->half_steps > 2) {
            const size_t kk = (size_t)B * p->kc * p->kc;
            L.C = off;
            off += align_up(sizeof(double) * kk);
            L.R1row = off;
            off += align_up(es * B * p->kc * p->c2);
            L.Sp = off;
            off += align_up(es * B * p->kc * p->c1);
            L.H = off;
            off += align_up(sizeof(float) * kk * dyra::kAlsGramSplit);
            L.Kp = off;
            off += align_up(sizeof(float) * kk);
        }
    } else if (path_for(p, n) == Path::Dual) {
        L.dual = off;
        off += align_up(dyra::decode_workspace_bytes(B, n, p->c1, p->c2, p->kw, p->kc));
    }
    L.total = off;
    return L;
}

// A row-major [rows][K] matrix (rows a multiple of 32, K of 16) in MFMA
// fragment order: the 32 x 16 block (row block rb, 16-deep step ks) is 512
// consecutive elements, lane l = 32 h + r of a wavefront holding row
// 32 rb + r, columns 16 ks + 8 h .. + 7.  Blocks follow each other step by
// step within a row block, so a wavefront that walks the contraction of one
// row block reads one contiguous run, 1 KB (bf16) per load instruction,
// each lane's piece already an MFMA operand.
std::vector<double> frag_tile(const std::vector<double> &src, int64_t rows, int64_t K) {
    std::vector<double> dst(src.size());
    const int64_t steps = K / 16;
    for (int64_t rb = 0; rb < rows / 32; ++rb)
        for (int64_t ks = 0; ks < steps; ++ks)
            for (int l = 0; l < 64; ++l) {
                const int64_t row = 32 * rb + (l & 31), col = 16 * ks + 8 * (l >> 5);
                double *d = &dst[(size_t)(((rb * steps + ks) * 64 + l) * 8)];
                for (int e = 0; e < 8; ++e) d[e] = src[(size_t)(row * K + col + e)];
            }
    return dst;
}

// A device copy of `src` rounded to `dtype` (round to nearest even); the
// current device receives it.
dyra_status upload_rounded(const std::vector<double> &src, dyra_dtype dtype, void **dst) {
    const size_t es = elem_size(dtype);
    const size_t bytes = std::max<size_t>(src.size() * es, 16);
    if (hipMalloc(dst, bytes) != hipSuccess) return DYRA_ERR_NOMEM;
    std::vector<unsigned char> host(bytes, 0);
    if (dtype == DYRA_BF16) {
        uint16_t *h = (uint16_t *)host.data();
        for (size_t i = 0; i < src.size(); ++i) h[i] = bf16_bits(src[i]);
    } else {
        float *h = (float *)host.data();
        for (size_t i = 0; i < src.size(); ++i) h[i] = (float)src[i];
    }
    return hipMemcpy(*dst, host.data(), bytes, hipMemcpyHostToDevice) == hipSuccess ? DYRA_OK : DYRA_ERR_HIP;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

dyra_status hip_status(hipError_t e) { return e == hipSuccess ? DYRA_OK : DYRA_ERR_HIP; }

// The kernels' one-time host set-up on the current device, done while
// preparing a plan so that forward calls only enqueue work.
dyra_status prepare_launches(dyra_dtype dtype, int device) {
    const dyra_status s = scratch_setup(device);
    if (s != DYRA_OK) return s;
    if (dtype == DYRA_BF16)
        return hip_status(dyra::gemm_prepare<bf16>()) == DYRA_OK ? hip_status(dyra::blast_prepare<bf16>())
                                                                 : DYRA_ERR_HIP;
    return hip_status(dyra::gemm_prepare<float>()) == DYRA_OK ? hip_status(dyra::blast_prepare<float>())
                                                              : DYRA_ERR_HIP;
}

dyra_status check_device(int device) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DYRA_ERR_NODEVICE;
    return cur == device ? DYRA_OK : DYRA_ERR_NODEVICE;
}

// Names of the kernels dyra_forward enqueues for (plan, n), in order.
std::vector<const char *> stage_list(const dyra_plan *p, int64_t n) {
    switch (path_for(p, n)) {
    case Path::Dual: return {"decode_project", "decode_coef", "decode_output"};
    case Path::Static:
        if (p->nb > 0) return {"left", "blast_mix", "output"};
        return {"left", "output"};
    case Path::Primal: break;
    }
    std::vector<const char *> v = {"left"};
    if (p->nb > 0) v.push_back("blast_mix");
    if (p->ns_iters > 0) {
        v.push_back("ns_factor");
        v.push_back("ns_apply");
    } else {
        v.push_back("gram_q");
    }
    v.push_back("mprime");
    v.push_back("right");
    for (int h = 2; h < p->half_steps; h += 2) {
        for (const char *st : {"als_transpose", "als_s", "als_gram", "als_coef", "als_lupdate"})
            v.push_back(st);
        if (h + 1 < p->half_steps)
            for (const char *st : {"gram_q", "mprime", "right"}) v.push_back(st);
    }
    v.push_back("output");
    return v;
}

template <typename E>
dyra_status run_forward(const E *X, int64_t B, int64_t n, const dyra_plan *p, const E *bias, float alpha, E *Y,
                        char *ws, const Layout &L, hipStream_t st, void *const *events, int32_t n_events,
                        int32_t *n_recorded) {
    int32_t ev = 0;
    const dyra::EventMark em{events, n_events, &ev, st};
    auto mark = [&]() -> dyra_status { return hip_status(em(hipSuccess)); };
    const int64_t N = B * n;
    const E *Aext = (const E *)p->Aext;
    const E *Vs = (const E *)p->Vs;
    const E *Wres_t = (const E *)p->Wres_t;
    int *flags = (int *)(ws + L.flags);
    dyra_status s;
    if ((s = mark()) != DYRA_OK) return s;
    const Path path = path_for(p, n);
    if (path != Path::Dual) {
        E *T = (E *)(ws + L.T);
        const int64_t ldt = p->kw + p->kc;
        if (p->nb == 0) {
            // T = X [A_s | P_L]^T: the static projection and L1 in one pass over X
            if ((s = hip_status(dyra::launch_gemm_store<E>(X, p->c1, Aext, p->c1, N, ldt, p->c1, T, ldt, st))) !=
                DYRA_OK)
                return s;
            if ((s = mark()) != DYRA_OK) return s;
        } else {
            // BLAST: Z_i = X_i U_i into T's block i, L1 = X P_L next to them,
            // then H_j = sum_i Z_i diag(s_ij) in place
            const int64_t pb = p->c1 / p->nb;
            const E *Ub = (const E *)p->Ublk;
            if (dyra::gemm_groupable(N, (int64_t)p->nb * p->rbp, p->rbp)) {
                // one launch: column group i reads X's columns from i * pb
                if ((s = hip_status(dyra::launch_gemm_store_grouped<E>(X, p->c1, Ub, pb, N, (int64_t)p->nb * p->rbp,
                                                                       pb, p->rbp, pb, T, ldt, st))) != DYRA_OK)
                    return s;
            } else {
                for (int i = 0; i < p->nb; ++i)
                    if ((s = hip_status(dyra::launch_gemm_store<E>(X + i * pb, p->c1, Ub + (int64_t)i * p->rbp * pb,
                                                                   pb, N, p->rbp, pb, T + (int64_t)i * p->rbp, ldt,
                                                                   st))) != DYRA_OK)
                        return s;
            }
            if (p->kc > 0 && (s = hip_status(dyra::launch_gemm_store<E>(X, p->c1, Aext, p->c1, N, p->kc, p->c1,
                                                                       T + p->kw, ldt, st))) != DYRA_OK)
                return s;
            if ((s = mark()) != DYRA_OK) return s;
            if ((s = hip_status(dyra::launch_blast_mix<E>(T, ldt, N, p->nb, p->rbp, (const float *)p->Smix, st))) !=
                DYRA_OK)
                return s;
            if ((s = mark()) != DYRA_OK) return s;
        }
        E *R1t = nullptr;
        if (path == Path::Primal) {
            E *Qt = (E *)(ws + L.Qt);
            E *Mp = (E *)(ws + L.Mp);
            R1t = (E *)(ws + L.R1t);
            double *Cf = p->half_steps > 2 ? (double *)(ws + L.C) : nullptr;
            // R update (Eq. 5, Algorithm 1 line 12): Q = L C^-T in place, M' = Q^T X,
            // R' = M' W_res (times alpha when it is the last update)
            auto r_update = [&](float alpha_r) -> dyra_status {
                dyra_status t;
                if (p->ns_iters > 0) {
                    if ((t = hip_status(dyra::launch_ns_solve<E>(T, ldt, p->kw, B, n, L.npad, p->k, p->kc, p->lambda,
                                                                 p->ns_iters, (float *)(ws + L.F), flags,
                                                                 p->dtype == DYRA_F32 ? (float *)Qt : nullptr, st,
                                                                 em))) != DYRA_OK)
                        return t;
                } else {
                    if ((t = hip_status(dyra::launch_gram_q<E>(T, ldt, p->kw, B, n, L.npad, p->k, p->kc, p->lambda,
                                                               Qt, (float *)(ws + L.Ct), (float *)(ws + L.Gw), flags,
                                                               Cf, st))) != DYRA_OK)
                        return t;
                    if ((t = mark()) != DYRA_OK) return t;
                }
                if ((t = hip_status(dyra::launch_mprime<E>(X, T, ldt, p->kw, Qt, B, n, L.npad, p->c1, p->kc, Mp,
                                                           st))) != DYRA_OK)
                    return t;
                if ((t = mark()) != DYRA_OK) return t;
                if ((t = hip_status(dyra::launch_right<E>(Mp, Wres_t, B * p->kc, p->c1, p->c2, p->kc, alpha_r, R1t,
                                                          st))) != DYRA_OK)
                    return t;
                return mark();
            };
            if ((s = r_update(p->half_steps == 2 ? alpha : 1.f)) != DYRA_OK) return s;
            // further ALS steps (§3.3 ablation): an L update (Eq. 4), then an R update
            for (int h = 2; h < p->half_steps; h += 2) {
                const bool last_l = h + 1 == p->half_steps;
                const dyra::AlsArgs<E> a{X, B, n, p->c1, p->c2, p->kc, p->k, p->lambda, R1t, (E *)(ws + L.R1row),
                                         (const E *)p->Wres, (E *)(ws + L.Sp), (float *)(ws + L.H), Cf,
                                         (float *)(ws + L.Kp), flags, T, ldt, p->kw};
                if ((s = hip_status(dyra::launch_als_lupdate<E>(a, last_l ? 1 : 0, alpha, st, em))) != DYRA_OK)
                    return s;
                if (last_l) break;
                if ((s = r_update(h + 2 == p->half_steps ? alpha : 1.f)) != DYRA_OK) return s;
            }
        }
        const int kc = path == Path::Primal ? p->kc : 0;
        if (p->nb == 0) {
            if ((s = hip_status(dyra::launch_output<E>(T, ldt, p->kw, kc, Vs, R1t, N, n, p->c2, bias, Y, st))) !=
                DYRA_OK)
                return s;
        } else {
            // BLAST: Y_j = H_j V_j^T + L1 R1_b[:, block j], one GEMM per block column
            const int64_t qb = p->c2 / p->nb;
            if (dyra::gemm_groupable(N, p->c2, (int)qb)) {
                // one launch: column group j reads H_j from T's column j * rbp
                if ((s = hip_status(dyra::launch_output_ex<E>(T, ldt, p->rbp, Vs, p->rbp, p->kw, kc, R1t,
                                                              p->c2 * p->kc, N, n, p->c2, bias, Y, p->c2, (int)qb,
                                                              p->rbp, st))) != DYRA_OK)
                    return s;
            } else {
                for (int j = 0; j < p->nb; ++j) {
                    const int64_t h0 = (int64_t)j * p->rbp;
                    if ((s = hip_status(dyra::launch_output_ex<E>(
                             T + h0, ldt, p->rbp, Vs + j * qb * p->rbp, p->rbp, (int)(p->kw - h0), kc,
                             R1t ? R1t + j * qb * p->kc : nullptr, p->c2 * p->kc, N, n, qb,
                             bias ? bias + j * qb : nullptr, Y + j * qb, p->c2, 0, 0, st))) != DYRA_OK)
                        return s;
                }
            }
        }
        if ((s = mark()) != DYRA_OK) return s;
    } else {
        dyra::DecodeArgs<E> a{X, B, n, p->c1, p->c2, p->kw, p->kc, p->k, p->lambda, (const E *)p->Adec,
                              (const E *)p->Vdec, (const E *)p->Wdec, Y,
                              ws + L.dual, flags, bias, alpha};
        if ((s = hip_status(dyra::launch_decode_project<E>(a, st))) != DYRA_OK) return s;
        if ((s = mark()) != DYRA_OK) return s;
        if ((s = hip_status(dyra::launch_decode_coef<E>(a, st))) != DYRA_OK) return s;
        if ((s = mark()) != DYRA_OK) return s;
        if ((s = hip_status(dyra::launch_decode_output<E>(a, st))) != DYRA_OK) return s;
        if ((s = mark()) != DYRA_OK) return s;
    }
    if (n_recorded) *n_recorded = ev;
    return DYRA_OK;
}

// Flags start at zero for every call: the per-instance failure flags are
// written (0 or 1) by the SPD-solve kernel for every instance, never accumulated.
dyra_status forward_impl(const void *X, int64_t B, int64_t n, const dyra_plan *p, const void *bias, float alpha,
                         void *Y, void *workspace, size_t workspace_bytes, void *stream, void *const *events,
                         int32_t n_events, int32_t *n_recorded) {
    if (n_recorded) *n_recorded = 0;
    if (!p) return DYRA_ERR_ARG;
    if (!std::isfinite(alpha)) return DYRA_ERR_ARG;
    if (bias && ((uintptr_t)bias % elem_size(p->dtype)) != 0) return DYRA_ERR_ALIGN;
    if (B < 0 || n < 1) return DYRA_ERR_SHAPE;
    if (B == 0) return DYRA_OK;
    if (!X || !Y) return DYRA_ERR_ARG;
    if (!aligned16(X) || !aligned16(Y)) return DYRA_ERR_ALIGN;
    if (B > INT32_MAX / std::max<int64_t>(n, 1)) return DYRA_ERR_SHAPE;
    const Path path = path_for(p, n);
    if (path == Path::Dual && n > kMaxWideDualTokens) return DYRA_ERR_SHAPE;  // n < k, lambda = 0, n > 64
    if (path == Path::Dual && p->half_steps > 2) return DYRA_ERR_SHAPE;   // one ALS step only in the dual form
    // BLAST plans solve the k x k system in every case: it is singular for
    // fewer tokens than k without a ridge term
    if (p->nb > 0 && p->kc > 0 && p->lambda == 0.f && n < p->k) return DYRA_ERR_SHAPE;
    const Layout L = workspace_layout(p, B, n);
    if (!workspace || workspace_bytes < L.total) return DYRA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DYRA_ERR_ALIGN;
    dyra_status s = check_device(p->device);
    if (s != DYRA_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    char *ws = (char *)workspace;
    if (p->dtype == DYRA_BF16)
        return run_forward<bf16>((const bf16 *)X, B, n, p, (const bf16 *)bias, alpha, (bf16 *)Y, ws, L, st, events,
                                 n_events, n_recorded);
    return run_forward<float>((const float *)X, B, n, p, (const float *)bias, alpha, (float *)Y, ws, L, st, events,
                              n_events, n_recorded);
}

}  // namespace

extern "C" {

const char *dyra_status_str(dyra_status s) {
    switch (s) {
    case DYRA_OK: return "ok";
    case DYRA_ERR_ARG: return "invalid argument";
    case DYRA_ERR_SHAPE: return "unsupported shape";
    case DYRA_ERR_DTYPE: return "unknown dtype";
    case DYRA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case DYRA_ERR_NUMERIC: return "numerical failure";
    case DYRA_ERR_HIP: return "HIP runtime error";
    case DYRA_ERR_NOMEM: return "out of memory";
    case DYRA_ERR_WORKSPACE: return "workspace missing or too small";
    case DYRA_ERR_NODEVICE: return "no device or wrong device";
    case DYRA_ERR_SCRATCH: return "call needs more than the built-in scratch of dyra_forward_noalloc";
    }
    return "unknown status";
}

dyra_status dyra_prepare(const float *W, int64_t c1, int64_t c2, int32_t r, int32_t k, float lambda,
                         dyra_dtype dtype, int device, dyra_plan **plan_out) {
    return dyra_prepare_ex(W, c1, c2, r, k, lambda, dtype, device, nullptr, 2, 0, plan_out);
}

dyra_status dyra_prepare_ex(const float *W, int64_t c1, int64_t c2, int32_t r, int32_t k, float lambda,
                            dyra_dtype dtype, int device, const float *R0, int32_t als_half_steps, int32_t ns_iters,
                            dyra_plan **plan_out) {
    if (!plan_out) return DYRA_ERR_ARG;
    *plan_out = nullptr;
    if (dtype != DYRA_BF16 && dtype != DYRA_F32) return DYRA_ERR_DTYPE;
    if (!W || c1 <= 0 || c2 <= 0 || r < 0 || k < 0) return DYRA_ERR_ARG;
    if (als_half_steps < 2 || als_half_steps > kMaxHalfSteps) return DYRA_ERR_ARG;
    if (ns_iters < 0 || ns_iters > kMaxNsIters) return DYRA_ERR_ARG;
    if (ns_iters > 0 && als_half_steps > 2) return DYRA_ERR_ARG;  // one ALS step with the Newton-Schulz solve
    if ((int64_t)r + k > std::min(c1, c2)) return DYRA_ERR_ARG;
    if (!(lambda >= 0.f) || !std::isfinite(lambda)) return DYRA_ERR_ARG;
    if (c1 % 32 != 0 || c2 % 32 != 0) return DYRA_ERR_SHAPE;
    if (k > kMaxCorrection) return DYRA_ERR_SHAPE;
    if (k > kMaxCorrectionSmall && (dtype == DYRA_F32 || als_half_steps > 2)) return DYRA_ERR_SHAPE;
    const int32_t kw = r > 0 ? (int32_t)round_up(r, 32) : 0;
    // the Newton-Schulz products of ranks above 64 run in 64-wide tiles
    const int32_t kc = k > 0 ? (int32_t)round_up(k, (ns_iters > 0 && k > kMaxCorrectionSmall) ? 64 : 16) : 0;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return DYRA_ERR_NODEVICE;

    dyra::Factors f;
    dyra_status s = dyra::factorize(W, c1, c2, r, k, (double)lambda, &f, k > 0 ? R0 : nullptr);
    if (s != DYRA_OK) return s;

    const size_t nA = (size_t)(kw + kc) * c1, nV = (size_t)c2 * kw, nR = (size_t)c2 * c1;
    std::vector<double> A(nA, 0.0), V(nV, 0.0), Rt(nR, 0.0);
    for (int64_t a = 0; a < c1; ++a) {
        for (int32_t i = 0; i < r; ++i) A[(size_t)i * c1 + a] = f.A_s[a * r + i];
        for (int32_t i = 0; i < k; ++i) A[(size_t)(kw + i) * c1 + a] = f.P_L[a * k + i];
    }
    for (int64_t b = 0; b < c2; ++b)
        for (int32_t i = 0; i < r; ++i) V[(size_t)b * kw + i] = f.V_s[b * r + i];
    for (int64_t a = 0; a < c1; ++a)
        for (int64_t b = 0; b < c2; ++b) Rt[(size_t)b * c1 + a] = f.W_res[a * c2 + b];

    dyra_plan *p = new (std::nothrow) dyra_plan{};
    if (!p) return DYRA_ERR_NOMEM;
    p->device = device;
    p->dtype = dtype;
    p->c1 = c1;
    p->c2 = c2;
    p->r = r;
    p->k = k;
    p->kw = kw;
    p->kc = kc;
    p->lambda = lambda;
    p->half_steps = k > 0 ? als_half_steps : 2;
    p->ns_iters = k > 0 ? ns_iters : 0;
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (hipSetDevice(device) != hipSuccess) {
        delete p;
        return DYRA_ERR_NODEVICE;
    }
    auto upload = [&](const std::vector<double> &src, void **dst) { return upload_rounded(src, dtype, dst); };
    if ((s = upload(A, &p->Aext)) == DYRA_OK && (s = upload(V, &p->Vs)) == DYRA_OK)
        s = upload(Rt, &p->Wres_t);
    if (s == DYRA_OK && p->half_steps > 2) s = upload(f.W_res, &p->Wres);
    if (s == DYRA_OK && kc > 0 && (s = upload(frag_tile(Rt, c2, c1), &p->Wdec)) == DYRA_OK &&
        (s = upload(frag_tile(V, c2, kw), &p->Vdec)) == DYRA_OK) {
        const int64_t rows = (kw + kc + 31) / 32 * 32;
        std::vector<double> Ap(A);
        Ap.resize((size_t)rows * c1, 0.0);
        s = upload(frag_tile(Ap, rows, c1), &p->Adec);
    }
    if (s == DYRA_OK) s = prepare_launches(dtype, device);
    if (prev >= 0) (void)hipSetDevice(prev);
    if (s != DYRA_OK) {
        dyra_plan_destroy(p);
        return s;
    }
    *plan_out = p;
    return DYRA_OK;
}

dyra_status dyra_prepare_blast(const float *W, int64_t c1, int64_t c2, int32_t nb, int32_t rb, const float *U,
                               const float *S, const float *V, int32_t k, float lambda, dyra_dtype dtype, int device,
                               dyra_plan **plan_out) {
    if (!plan_out) return DYRA_ERR_ARG;
    *plan_out = nullptr;
    if (dtype != DYRA_BF16 && dtype != DYRA_F32) return DYRA_ERR_DTYPE;
    if (!W || !U || !S || !V || c1 <= 0 || c2 <= 0 || nb < 1 || rb < 1 || k < 0) return DYRA_ERR_ARG;
    if (k > std::min(c1, c2)) return DYRA_ERR_ARG;
    if (!(lambda >= 0.f) || !std::isfinite(lambda)) return DYRA_ERR_ARG;
    if (nb > kMaxBlastBlocks) return DYRA_ERR_SHAPE;
    if (c1 % (32 * (int64_t)nb) != 0 || c2 % (32 * (int64_t)nb) != 0) return DYRA_ERR_SHAPE;
    if (k > kMaxCorrection) return DYRA_ERR_SHAPE;
    if (k > kMaxCorrectionSmall && dtype == DYRA_F32) return DYRA_ERR_SHAPE;
    const int32_t rbp = (int32_t)round_up(rb, 32);
    if ((int64_t)rbp * (int64_t)elem_size(dtype) > 16 * 256) return DYRA_ERR_SHAPE;  // the mix kernel's row chunks
    const int32_t kc = k > 0 ? (int32_t)round_up(k, 16) : 0;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) return DYRA_ERR_NODEVICE;

    dyra::Factors f;
    dyra_status s = dyra::factorize_blast(W, c1, c2, nb, rb, U, S, V, k, (double)lambda, &f);
    if (s != DYRA_OK) return s;

    const int64_t pb = c1 / nb;
    std::vector<double> Ub((size_t)nb * rbp * pb, 0.0), Vp((size_t)c2 * rbp, 0.0), Pt((size_t)kc * c1, 0.0),
        Rt((size_t)c2 * c1, 0.0);
    std::vector<float> Sm((size_t)nb * nb * rbp, 0.f);
    for (int64_t a = 0; a < c1; ++a) {
        const int64_t i = a / pb, ai = a % pb;
        for (int32_t c = 0; c < rb; ++c) Ub[((size_t)i * rbp + c) * pb + ai] = U[a * rb + c];
        for (int32_t c = 0; c < k; ++c) Pt[(size_t)c * c1 + a] = f.P_L[a * k + c];
    }
    for (int64_t b = 0; b < c2; ++b)
        for (int32_t c = 0; c < rb; ++c) Vp[(size_t)b * rbp + c] = V[b * rb + c];
    for (int64_t ij = 0; ij < (int64_t)nb * nb; ++ij)
        for (int32_t c = 0; c < rb; ++c) Sm[(size_t)ij * rbp + c] = S[ij * rb + c];
    for (int64_t a = 0; a < c1; ++a)
        for (int64_t b = 0; b < c2; ++b) Rt[(size_t)b * c1 + a] = f.W_res[a * c2 + b];

    dyra_plan *p = new (std::nothrow) dyra_plan{};
    if (!p) return DYRA_ERR_NOMEM;
    p->device = device;
    p->dtype = dtype;
    p->c1 = c1;
    p->c2 = c2;
    p->r = rb;
    p->k = k;
    p->kw = nb * rbp;
    p->kc = kc;
    p->lambda = lambda;
    p->half_steps = 2;
    p->ns_iters = 0;
    p->nb = nb;
    p->rbp = rbp;
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (hipSetDevice(device) != hipSuccess) {
        delete p;
        return DYRA_ERR_NODEVICE;
    }
    if ((s = upload_rounded(Ub, dtype, &p->Ublk)) == DYRA_OK && (s = upload_rounded(Vp, dtype, &p->Vs)) == DYRA_OK &&
        (s = upload_rounded(Pt, dtype, &p->Aext)) == DYRA_OK)
        s = upload_rounded(Rt, dtype, &p->Wres_t);
    if (s == DYRA_OK) {
        if (hipMalloc(&p->Smix, Sm.size() * sizeof(float)) != hipSuccess) s = DYRA_ERR_NOMEM;
        else if (hipMemcpy(p->Smix, Sm.data(), Sm.size() * sizeof(float), hipMemcpyHostToDevice) != hipSuccess)
            s = DYRA_ERR_HIP;
    }
    if (s == DYRA_OK) s = prepare_launches(dtype, device);
    if (prev >= 0) (void)hipSetDevice(prev);
    if (s != DYRA_OK) {
        dyra_plan_destroy(p);
        return s;
    }
    *plan_out = p;
    return DYRA_OK;
}

void dyra_plan_destroy(dyra_plan *plan) {
    if (!plan) return;
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(plan->device);
    if (plan->Aext) (void)hipFree(plan->Aext);
    if (plan->Vs) (void)hipFree(plan->Vs);
    if (plan->Wres_t) (void)hipFree(plan->Wres_t);
    if (plan->Wres) (void)hipFree(plan->Wres);
    if (plan->Wdec) (void)hipFree(plan->Wdec);
    if (plan->Vdec) (void)hipFree(plan->Vdec);
    if (plan->Adec) (void)hipFree(plan->Adec);
    if (plan->Ublk) (void)hipFree(plan->Ublk);
    if (plan->Smix) (void)hipFree(plan->Smix);
    if (prev >= 0) (void)hipSetDevice(prev);
    delete plan;
}

dyra_status dyra_plan_info(const dyra_plan *p, int64_t *c1, int64_t *c2, int32_t *r, int32_t *k, float *lambda,
                           dyra_dtype *dtype, int *device) {
    if (!p) return DYRA_ERR_ARG;
    if (c1) *c1 = p->c1;
    if (c2) *c2 = p->c2;
    if (r) *r = p->r;
    if (k) *k = p->k;
    if (lambda) *lambda = p->lambda;
    if (dtype) *dtype = p->dtype;
    if (device) *device = p->device;
    return DYRA_OK;
}

size_t dyra_workspace_bytes(const dyra_plan *plan, int64_t B, int64_t n) {
    if (!plan || B < 0 || n < 1) return 0;
    return workspace_layout(plan, B, n).total;
}

dyra_status dyra_forward(const void *X, int64_t B, int64_t n, const dyra_plan *plan, void *Y, void *workspace,
                         size_t workspace_bytes, void *stream) {
    return forward_impl(X, B, n, plan, nullptr, 1.f, Y, workspace, workspace_bytes, stream, nullptr, 0, nullptr);
}

dyra_status dyra_forward_ex(const void *X, int64_t B, int64_t n, const dyra_plan *plan, const void *bias,
                            float alpha, void *Y, void *workspace, size_t workspace_bytes, void *stream) {
    return forward_impl(X, B, n, plan, bias, alpha, Y, workspace, workspace_bytes, stream, nullptr, 0, nullptr);
}

dyra_status dyra_forward_timed(const void *X, int64_t B, int64_t n, const dyra_plan *plan, void *Y,
                               void *workspace, size_t workspace_bytes, void *stream, void *const *events,
                               int32_t n_events, int32_t *n_recorded) {
    if (!events || n_events < 1) return DYRA_ERR_ARG;
    return forward_impl(X, B, n, plan, nullptr, 1.f, Y, workspace, workspace_bytes, stream, events, n_events,
                        n_recorded);
}

dyra_status dyra_forward_noalloc(const void *X, int64_t B, int64_t n, const dyra_plan *plan, void *Y,
                                 void *stream) {
    if (!plan) return DYRA_ERR_ARG;
    if (B < 0 || n < 1) return DYRA_ERR_SHAPE;
    if (B == 0) return DYRA_OK;
    const size_t need = dyra_workspace_bytes(plan, B, n);
    if (need > kNoallocScratchBytes) return DYRA_ERR_SCRATCH;
    void *ws = scratch_ptr(plan->device);
    if (!ws) return DYRA_ERR_NODEVICE;
    return forward_impl(X, B, n, plan, nullptr, 1.f, Y, ws, kNoallocScratchBytes, stream, nullptr, 0, nullptr);
}

size_t dyra_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

const char *dyra_stage_name(const dyra_plan *plan, int64_t n, int32_t i) {
    if (!plan || n < 1 || i < 0) return nullptr;
    const std::vector<const char *> v = stage_list(plan, n);
    return i < (int32_t)v.size() ? v[(size_t)i] : nullptr;
}

dyra_status dyra_forward_status(const dyra_plan *plan, int64_t B, int64_t n, const void *workspace, void *stream,
                                int32_t *failures) {
    if (!plan || !workspace || !failures || B < 0 || n < 1) return DYRA_ERR_ARG;
    *failures = 0;
    // the weight-only path solves nothing and writes no flag
    if (B == 0 || path_for(plan, n) == Path::Static) return DYRA_OK;
    const Layout L = workspace_layout(plan, B, n);
    std::vector<int32_t> flags((size_t)B);
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(flags.data(), (const char *)workspace + L.flags, sizeof(int32_t) * (size_t)B,
                       hipMemcpyDeviceToHost, st) != hipSuccess)
        return DYRA_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return DYRA_ERR_HIP;
    int32_t c = 0;
    for (int32_t f : flags) c += f != 0;
    *failures = c;
    return DYRA_OK;
}

dyra_status dyra_dense_ref(const void *X, const void *Wt, int64_t N, int64_t c1, int64_t c2, dyra_dtype dtype,
                           void *Y, void *stream) {
    if (dtype != DYRA_BF16 && dtype != DYRA_F32) return DYRA_ERR_DTYPE;
    if (N < 0 || c1 <= 0 || c2 <= 0) return DYRA_ERR_SHAPE;
    if (c1 % 32 != 0 || c2 % 32 != 0) return DYRA_ERR_SHAPE;
    if (N == 0) return DYRA_OK;
    if (!X || !Wt || !Y) return DYRA_ERR_ARG;
    if (!aligned16(X) || !aligned16(Wt) || !aligned16(Y)) return DYRA_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == DYRA_BF16)
        return hip_status(dyra::launch_gemm_store<bf16>((const bf16 *)X, c1, (const bf16 *)Wt, c1, N, c2, c1,
                                                        (bf16 *)Y, c2, st));
    return hip_status(
        dyra::launch_gemm_store<float>((const float *)X, c1, (const float *)Wt, c1, N, c2, c1, (float *)Y, c2, st));
}

}  // extern "C"
