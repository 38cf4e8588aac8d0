// Tiled MFMA GEMM for gfx950: D = A B^T with both operands K-contiguous.
//
// Used for the exact product X W (the dense reference, §2.1 Eq. 2), the left
// pass T = X [A_s | P_L] that yields both the static projection X A_s and the
// left factor L1 = X P_L (DyRA paper Eq. 7), the stacked right factor
// R1 = M' W_res of all instances at once (Eq. 5; the O(c1 c2 r) term of §2.3)
// and the output Y = (X A_s) V_s^T + L1 R1_b (Eq. 6 with Proposition 1's
// factored static part).
//
// A workgroup owns a BM x BN output tile and its WM x WN wavefronts each own a
// (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks.  K advances in slices of SB
// bytes per operand row: 128 (whole cache lines) or, for float32 256 x 256
// tiles, 64.  Slices move from global memory straight into LDS
// (global_load_lds_dwordx4, no register staging), NS of them in flight, so a
// slice's loads have NS - 1 slices of MFMA work to land; one barrier per slice.
// In LDS a slice row is SB / 16 chunks of 16 bytes, swizzled so that the 16
// rows a quarter wavefront reads with ds_read_b128 fall on distinct banks.  Tiles
// are handed out XCD by XCD: workgroup ids are dealt round-robin over the 8
// XCDs, so id i works on tile (i % 8) * ceil(T/8) + i / 8 and each XCD's L2
// sees a contiguous band of tiles that share operand panels.
//
// The output product appends correction slices to the K loop: for every
// instance b whose tokens fall in the tile, A's correction columns (the rows of
// Q_b; rows of other instances are zeroed in registers) meet R1_b, so each
// token row picks up exactly its own instance's L1 R1_b in the same
// accumulators before Y is stored once (the fused merge of §2.4).  32-row
// blocks with no token of b skip those MFMAs.
#include "dyra_kernels.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "mfma_tile.h"

namespace dyra {

namespace {

// One K slice is SB bytes of every operand row: 128 (whole cache lines) or 64
// (shapes whose registers cannot hold the fragments of 128 plus their
// accumulators).
template <typename E, int SB> constexpr int gemm_bk() { return SB / (int)sizeof(E); }

// MFMA operand fragment of 16-deep step h from a swizzled LDS slice row
// (row_base = the row's first byte, sw = the row's chunk swizzle, hf = lane / 32).
__device__ __forceinline__ bf16x8 slice_frag(const char *row_base, int h, int hf, int sw, const bf16 *) {
    return *reinterpret_cast<const bf16x8 *>(row_base + (((2 * h + hf) ^ sw) << 4));
}
__device__ __forceinline__ f32x8 slice_frag(const char *row_base, int h, int hf, int sw, const float *) {
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(row_base + (((4 * h + 2 * hf) ^ sw) << 4));
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(row_base + (((4 * h + 2 * hf + 1) ^ sw) << 4));
    f32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}


// Four consecutive elements packed for one 8-byte (bf16) / 16-byte (fp32) store.
template <typename E> struct Pack4;
template <> struct Pack4<bf16> { typedef uint2 type; };
template <> struct Pack4<float> { typedef uint4 type; };

template <typename E> __device__ __forceinline__ typename Pack4<E>::type pack4(const float (&v)[4]) {
    if constexpr (sizeof(E) == 2) {
        union { uint2 u; bf16 e[4]; } w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w.e[q] = to_elem<E>(v[q]);
        return w.u;
    } else {
        return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    }
}

// Epilogue functors.  fix4(v, i, j, ct) adjusts four float32 results before
// they are rounded to E: (i, j) is the first of four consecutive columns of row
// i (row-major stores) or of four consecutive rows of column j (R1t stores);
// ct, for functors with kColumnTerms, points at the four columns' additive
// terms as the kernel staged them in LDS (null when there are none).  store4
// then writes the rounded four.

// Row-major D: store4(i, j, p) writes columns j..j+3 of row i, as a
// non-temporal store (the outputs of these products are not read again by the
// kernel; streaming them keeps them from evicting cached operands).  With a bias
// (the fused linear layer of §2.4: Y = X_tmp A^T + b + alpha L R) every row
// gets bias[j] added to column j before rounding; the kernel reads the tile's
// bias columns once per tile into LDS (read per element from global memory,
// each of the epilogue's loads waited in turn and cost more than the tile's
// MFMAs).
template <typename E> struct RowStore {
    static constexpr bool kColumnTerms = true;
    E *D;
    int64_t ldd;
    const E *bias = nullptr;  // [ncols] or null
    int64_t ncols = 0;
    __device__ __forceinline__ void fix4(float (&v)[4], int64_t, int64_t, const float *ct) const {
        if (ct) {
            const f32x4 b = *reinterpret_cast<const f32x4 *>(ct);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] += b[q];
        }
    }
    __device__ __forceinline__ void store4(int64_t i, int64_t j, const typename Pack4<E>::type &p) const {
        if constexpr (sizeof(E) == 2) {
            typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
            const u32x2v v = {p.x, p.y};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2v *>(D + i * ldd + j));
        } else {
            const u32x4 v = {p.x, p.y, p.z, p.w};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(D + i * ldd + j));
        }
    }
};

// Stacked right factor: rows r..r+3 (= correction indices kk..kk+3 of
// instance b = r / kc) of column c, stored as R1t[b][c][kk..kk+3], scaled by
// alpha (the correction's weight in §2.4's fused output; 1 in Eq. 6).
template <typename E> struct R1tStore {
    static constexpr bool kColumnTerms = false;
    E *R1t;
    int64_t kc, c2;
    float alpha = 1.f;
    __device__ __forceinline__ void fix4(float (&v)[4], int64_t, int64_t, const float *) const {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] *= alpha;
    }
    __device__ __forceinline__ void store4(int64_t r, int64_t c, const typename Pack4<E>::type &p) const {
        // rows are below 2^31 (instances x correction rank): 32-bit division
        const uint32_t ru = (uint32_t)r, kcu = (uint32_t)kc;
        const int64_t b = ru / kcu, kk = ru - (uint32_t)b * kcu;
        *reinterpret_cast<typename Pack4<E>::type *>(R1t + (b * c2 + c) * kc + kk) = p;
    }
};

constexpr size_t kLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950

template <int BM, int BN, int NS, int SB> constexpr size_t stage_bytes() { return (size_t)NS * (BM + BN) * SB; }
// LDS of the staged epilogue: the whole tile as [BM][BN + 4] (ROWS) or
// [BN][BM + 4] elements; tiles that do not fit store straight from registers.
template <typename E, int BM, int BN, bool ROWS> constexpr size_t epi_bytes() {
    return ROWS ? sizeof(E) * (size_t)BM * (BN + 4) : sizeof(E) * (size_t)BN * (BM + 4);
}
template <typename E, int BM, int BN, bool ROWS> constexpr bool epi_staged() {
    return epi_bytes<E, BM, BN, ROWS>() <= kLdsBytes;
}

// Correction slices of the output product (unused when CORR is false):
// instance b's Q_b sits in columns [kcol, kcol + kc) of A's rows b*n ..
// b*n + n - 1, and its R1_b is the [N][kc] matrix R1t + b * N * kc.
template <typename E> struct Corr {
    const E *R1t;
    int64_t n;
    int kcol, kc;
    int64_t rstride;  // elements from one instance's R1t block to the next
    // Grouped A operand (any kernel): output columns [g*gcols, g*gcols + gcols)
    // read A from column g*gstride on (each tile lies in one group); gcols = 0
    // for none.  The correction columns stay at kcol from A itself.
    int gcols = 0;
    int64_t gstride = 0;
};

template <typename E, int BM, int BN, int NS, int SB, bool ROWS> constexpr size_t gemm_smem() {
    return (epi_staged<E, BM, BN, ROWS>() && epi_bytes<E, BM, BN, ROWS>() > stage_bytes<BM, BN, NS, SB>())
               ? epi_bytes<E, BM, BN, ROWS>()
               : stage_bytes<BM, BN, NS, SB>();
}
// ... plus BN floats of per-column terms after it for functors that have them
template <typename E, int BM, int BN, int NS, int SB, bool ROWS, class Epi> constexpr size_t gemm_smem_total() {
    return gemm_smem<E, BM, BN, NS, SB, ROWS>() + (Epi::kColumnTerms ? sizeof(float) * BN : 0);
}

// ROWS = true: the epilogue receives four consecutive columns of one row (the
// MFMA is issued with the operands swapped, so a lane holds a row of the
// block); ROWS = false: four consecutive rows of one column.  K must be a
// multiple of 16 (a last slice may be short).
template <typename E, int BM, int BN, int WM, int WN, int NS, int SB, bool ROWS, bool CORR, class Epi,
          bool GROUPED>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const E *__restrict__ A, int64_t lda,
                                                            const E *__restrict__ B, int64_t ldb, int64_t M,
                                                            int64_t N, int64_t K, int tiles_n, int ntiles,
                                                            int per_xcd, Corr<E> corr, Epi epi) {
    constexpr int NW = WM * WN;
    constexpr int NT = 64 * NW;
    constexpr int BK = gemm_bk<E, SB>();
    constexpr int RPB = 1024 / SB;  // rows per 1 KB load block
    static_assert(SB == 64 || SB == 128, "slice bytes");
    constexpr int VEC = 16 / (int)sizeof(E);
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int IA = BM / RPB, ITOT = (BM + BN) / RPB;  // 1 KB load blocks per slice
    constexpr int IPW = (ITOT + NW - 1) / NW, IMIN = ITOT / NW;
    constexpr int STAGE = (BM + BN) * SB;  // bytes per slice
    constexpr int KSTEPS = BK / 16;         // 16-deep MFMA steps per slice
    static_assert(TM >= 1 && TN >= 1 && IMIN >= 1 && NS >= 2 && NS <= 4 && NW % 2 == 0, "tile shape");
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 31, hf = lane >> 5;
    // Slice row r holds chunk c at position c ^ sw(r): the 16 rows a quarter
    // wavefront reads with ds_read_b128 then fall on distinct banks.
    //   SB = 128: sw(r) = (r >> 1) & 7.  A load block is 8 rows; lane l fills
    //     position l % 8 of row l / 8, so block j's lane l fetches chunk
    //     (l % 8) ^ ((4 j + l / 16) % 8); j and the wavefront have the same
    //     parity (the wavefront count is even): one column per lane.
    //   SB = 64: sw(r) = (r >> 2) & 3.  A load block is 16 rows; lane l fills
    //     position l % 4 of row l / 4 and fetches chunk (l % 4) ^ ((l / 16) % 4).
    const int sw = SB == 128 ? (lr >> 1) & 7 : (lr >> 2) & 3;  // swizzle of the rows this lane reads
    const int frow = SB == 128 ? lane >> 3 : lane >> 2;
    const int fcol = (SB == 128 ? ((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7))
                                : ((lane & 3) ^ ((lane >> 4) & 3))) * VEC;
    // persistent: workgroup i runs on XCD i % 8 and walks that XCD's band of
    // tiles; the stores of one tile drain while the next tile computes
    const int xcd = (int)(blockIdx.x % 8), slot = (int)(blockIdx.x / 8), nslots = (int)(gridDim.x / 8);
    for (int tl = slot; tl < per_xcd; tl += nslots) {
    const int tile = xcd * per_xcd + tl;
    if (tile >= ntiles) break;
    const int64_t row0 = (int64_t)(tile / tiles_n) * BM;
    const int64_t col0 = (int64_t)(tile % tiles_n) * BN;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
    // the tile's per-column terms, requested now (ahead of the K slices' loads,
    // so they have landed by the first slice) and staged in LDS at the epilogue
    float cterm = 0.f;
    if constexpr (Epi::kColumnTerms) {
        static_assert(ROWS, "per-column terms with row-major stores");
        if (epi.bias != nullptr && tid < BN) {
            const int64_t c = col0 + tid;
            cterm = c < epi.ncols ? to_f32(epi.bias[c]) : 0.f;
        }
    }

    // static slices, then SC correction slices per instance of the tile
    const int64_t S0 = (K + BK - 1) / BK;
    const int tail_steps = (int)(K % BK) / 16;  // 16-deep steps of a short last static slice
    int64_t S = S0, b_first = 0;
    int SC = 1;
    if constexpr (CORR) {
        const int64_t rend = row0 + BM < M ? row0 + BM : M;
        b_first = row0 / corr.n;
        SC = (corr.kc + BK - 1) / BK;
        S = S0 + ((rend - 1) / corr.n - b_first + 1) * SC;
    }
    // Correction slices come in order (instance b_first + bi, slice sc of its
    // SC); both the loads and the MFMAs walk them in order, so each side
    // carries its (bi, sc) as a counter rather than dividing s - S0 by SC.
    struct CorrPos {
        int bi = 0, sc = 0;
        __device__ void next(int SCn) {
            if (++sc == SCn) {
                sc = 0;
                ++bi;
            }
        }
    } ipos, cpos;
    // instance b of position q and its token rows [rlo, rhi)
    auto inst_of = [&](const CorrPos &q, int64_t &b, int64_t &rlo, int64_t &rhi) {
        b = b_first + q.bi;
        rlo = b * corr.n;
        rhi = rlo + corr.n < M ? rlo + corr.n : M;
    };
    // static-slice source of this wave's q-th load block (rows clamped into
    // range: rows past M or N are computed and never stored).  For SB = 64 the
    // lane's column is folded in here; SB = 128 adds it per slice (each form
    // measured faster for its shapes).
    constexpr int64_t FC_IN_BASE = SB == 64;
    int64_t aoff = 0;  // grouped A operand: this tile's group offset (a template switch: the
                       // extra registers made the ungrouped correction kernels spill)
    if constexpr (GROUPED) aoff = (int64_t)((int)col0 / corr.gcols) * corr.gstride;
    const E *base[IPW];
#pragma unroll
    for (int q = 0; q < IPW; ++q) {
        const int j = wave + q * NW;
        if (j < IA) {
            const int64_t r = row0 + RPB * j + frow;
            base[q] = A + (r < M ? r : M - 1) * lda + aoff + (FC_IN_BASE ? fcol : 0);
        } else {
            const int64_t r = col0 + RPB * (j - IA) + frow;
            base[q] = B + (r < N ? r : N - 1) * ldb + (FC_IN_BASE ? fcol : 0);
        }
    }
    auto issue = [&](int64_t s) {
        char *dst = smem + (int)(s % NS) * STAGE;
        if (!CORR || s < S0) {
            // a K tail shorter than the slice fetches its missing columns from
            // column 0; they meet no MFMA
            int64_t off;
            if constexpr (FC_IN_BASE) {
                off = (s + 1) * BK <= K ? s * BK : (s * BK + fcol < K ? s * BK : -(int64_t)fcol);
            } else {
                const int64_t kc0 = s * BK + fcol;
                off = kc0 < K ? kc0 : 0;
            }
#pragma unroll
            for (int q = 0; q < IPW; ++q) {
                const int j = wave + q * NW;
                if (q < IMIN || j < ITOT) lds_dma16(base[q] + off, dst + j * 1024);
            }
        } else {
            int64_t b, rlo, rhi;
            inst_of(ipos, b, rlo, rhi);
            const int sc = ipos.sc;
            ipos.next(SC);
            int kl = sc * BK + fcol;
            kl = kl < corr.kc ? kl : 0;  // columns past kc are fetched from column 0 and never used
            // A rows: the static source shifted to Q's columns; B rows: R1_b
            const int64_t offA = corr.kcol + kl - (FC_IN_BASE ? fcol : 0) - (GROUPED ? aoff : 0);
            const E *gB = corr.R1t + b * corr.rstride + kl;
#pragma unroll
            for (int q = 0; q < IPW; ++q) {
                const int j = wave + q * NW;
                if (!(q < IMIN || j < ITOT)) continue;
                const E *g;
                if (j < IA) {
                    g = base[q] + offA;
                } else {
                    // (32-bit: N counts output features, N * kc < 2^31)
                    const int r = (int)col0 + RPB * (j - IA) + frow;
                    g = gB + (int64_t)((r < N ? r : (int)N - 1) * corr.kc);
                }
                lds_dma16(g, dst + j * 1024);
            }
        }
    };

    for (int64_t p = 0; p < NS - 1 && p < S; ++p) issue(p);
    // One K slice.  CS: a correction slice (instance rows masked, possibly
    // fewer 16-deep steps); the static slices are compiled without any of
    // that, as one run of MFMAs.
    auto slice = [&](int64_t s, auto KS) __attribute__((always_inline)) {
        constexpr int KIND = decltype(KS)::value;  // 0 static, 1 short last static slice, 2 correction
        constexpr bool CSL = KIND == 2;
        // this wave's loads of slice s have landed once at most `later` slices'
        // worth (issued after it) are outstanding; the barrier then makes every
        // wave's part visible and frees the buffer of slice s - 1
        const int64_t later = (S - 1 - s) < (NS - 2) ? (S - 1 - s) : (NS - 2);
        if (later >= 2) wait_vmcnt<2 * IMIN>();
        else if (later == 1) wait_vmcnt<IMIN>();
        else wait_vmcnt<0>();
        barrier_only();
        if (s + NS - 1 < S) issue(s + NS - 1);

        int ksteps = KIND == 1 ? tail_steps : KSTEPS;
        uint32_t live = ~0u;
        int64_t rlo = 0, rhi = 0;
        if constexpr (CSL) {
            int64_t b;
            inst_of(cpos, b, rlo, rhi);
            const int sc = cpos.sc;
            cpos.next(SC);
            const int kleft = (corr.kc - sc * BK) / 16;
            ksteps = kleft < KSTEPS ? kleft : KSTEPS;
            live = 0;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int64_t rb = row0 + (wm * TM + i) * 32;
                live |= (rb < rhi && rb + 32 > rlo) ? (1u << i) : 0u;
            }
        }
        const char *sa = smem + (int)(s % NS) * STAGE + ((wm * TM) * 32 + lr) * SB;
        const char *sb = smem + (int)(s % NS) * STAGE + BM * SB + ((wn * TN) * 32 + lr) * SB;
        // the fragments of two 16-deep steps are requested before their first
        // MFMA, so each pair waits on LDS latency once
        // (the 256 x 256 correction kernel reads one step at a time: two
        // steps' fragments do not fit beside its accumulators and addresses)
        constexpr int KG = (CORR && SB == 128 && BM * BN >= 65536) ? 1 : (KSTEPS < 2 ? KSTEPS : 2);
#pragma unroll
        for (int h0 = 0; h0 < KSTEPS; h0 += KG) {
            if (KIND != 0 && h0 >= ksteps) break;
            typename Frag<E>::type fa[KG][TM], fb[KG][TN];
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                const int h = h0 + g;
                if (KIND != 0 && h >= ksteps) break;
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[g][j] = slice_frag(sb + j * 32 * SB, h, hf, sw, (const E *)nullptr);
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[g][i] = slice_frag(sa + i * 32 * SB, h, hf, sw, (const E *)nullptr);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < KG; ++g) {
                if (KIND != 0 && h0 + g >= ksteps) break;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    typename Frag<E>::type a = fa[g][i];
                    if constexpr (CSL) {
                        if (!((live >> i) & 1u)) continue;
                        const int64_t r = row0 + (wm * TM + i) * 32 + lr;
                        if (!(r >= rlo && r < rhi)) a = zero_frag(a);
                    }
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = ROWS ? mma16(acc[i][j], fb[g][j], a) : mma16(acc[i][j], a, fb[g][j]);
                }
            }
        }
    };
    int64_t s = 0;
    for (; s < S0 - (tail_steps ? 1 : 0); ++s) slice(s, std::integral_constant<int, 0>{});
    if (tail_steps) slice(s++, std::integral_constant<int, 1>{});
    if constexpr (CORR) {
        for (; s < S; ++s) slice(s, std::integral_constant<int, 2>{});
    }
    float *const cts = reinterpret_cast<float *>(smem + gemm_smem<E, BM, BN, NS, SB, ROWS>());
    bool has_ct = false;
    if constexpr (Epi::kColumnTerms) {
        has_ct = epi.bias != nullptr;
        if (has_ct && tid < BN) cts[tid] = cterm;
    }
    __syncthreads();
    // ---- epilogue.  A lane holds four consecutive elements of the store's
    // contiguous direction (columns for ROWS, rows otherwise).  When the tile
    // fits in LDS it is staged there and written out with consecutive lanes on
    // consecutive addresses; otherwise each lane stores its own runs.
    constexpr int OR = ROWS ? BM : BN, OC = ROWS ? BN : BM;  // LDS tile [OR][OC + 4]
    constexpr int OS = OC + 4;
    E *const lds = reinterpret_cast<E *>(smem);
    if constexpr (epi_staged<E, BM, BN, ROWS>()) {
        typedef typename Pack4<E>::type P;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                  acc[i][j][4 * g + 3]};
                    const int ti = (wm * TM + i) * 32, tj = (wn * TN + j) * 32;
                    const int lrow = ROWS ? ti + lr : tj + lr;              // LDS row
                    const int lcol = (ROWS ? tj : ti) + acc_row(lane, 4 * g);  // 4 consecutive
                    epi.fix4(v, row0 + (ROWS ? lrow : lcol), col0 + (ROWS ? lcol : lrow), has_ct ? cts + lcol : nullptr);
                    *reinterpret_cast<P *>(lds + lrow * OS + lcol) = pack4<E>(v);
                }
        __syncthreads();
        constexpr int CPR = OC / 4, CH = OR * CPR;
#pragma unroll 4
        for (int c = tid; c < CH; c += NT) {
            const int orow = c / CPR, ocol = (c % CPR) * 4;
            const P v = *reinterpret_cast<const P *>(lds + orow * OS + ocol);
            const int64_t r = row0 + (ROWS ? orow : ocol), cc = col0 + (ROWS ? ocol : orow);
            if (r < M && cc < N) epi.store4(r, cc, v);
        }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                  acc[i][j][4 * g + 3]};
                    const int64_t rb = row0 + wm * TM * 32 + i * 32, cb0 = col0 + wn * TN * 32 + j * 32;
                    const int64_t r = ROWS ? rb + lr : rb + acc_row(lane, 4 * g);
                    const int64_t c = ROWS ? cb0 + acc_row(lane, 4 * g) : cb0 + lr;
                    epi.fix4(v, r, c, has_ct ? cts + (c - col0) : nullptr);
                    if (r < M && c < N) epi.store4(r, c, pack4<E>(v));
                }
    }
    // the epilogue's LDS reads finish before the next tile's loads land there
    __syncthreads();
    }
}


// One-time host set-up of a kernel instantiation on the current device: its
// dynamic LDS limit and the number of workgroups resident per CU (the
// persistent grid's size).  Done once per device under a lock, normally from
// the preparation calls (gemm_prepare), so that a forward call only launches.
struct LaunchSetup {
    std::mutex mu;
    std::atomic<uint64_t> done{0};  // bit d: device d is set up
    std::atomic<int> per_cu{0};     // the same on every gfx950 device
};

template <class K>
hipError_t ensure_setup(LaunchSetup &ls, K kfn, int threads, size_t smem) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
    if (bit && (ls.done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    std::lock_guard<std::mutex> lock(ls.mu);
    if (bit && (ls.done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute((const void *)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kfn, threads, smem);
    if (e != hipSuccess) return e;
    ls.per_cu.store(occ > 0 ? occ : 1, std::memory_order_relaxed);
    ls.done.fetch_or(bit, std::memory_order_release);
    return hipSuccess;
}

// setup_only: run the one-time set-up of this instantiation and launch nothing.
template <typename E, int BM, int BN, int WM, int WN, int NS, int SB, bool ROWS, bool CORR, bool GROUPED,
          class Epi>
hipError_t gemm_launch(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                       const Corr<E> &corr, Epi epi, hipStream_t st, bool setup_only = false) {
    static_assert(gemm_smem_total<E, BM, BN, NS, SB, ROWS, Epi>() <= kLdsBytes, "LDS");
    auto kfn = gemm_kernel<E, BM, BN, WM, WN, NS, SB, ROWS, CORR, Epi, GROUPED>;
    constexpr size_t smem = gemm_smem_total<E, BM, BN, NS, SB, ROWS, Epi>();
    static LaunchSetup ls;
    hipError_t e = ensure_setup(ls, kfn, 64 * WM * WN, smem);
    if (e != hipSuccess || setup_only) return e;
    if (K % 16 != 0) return hipErrorInvalidValue;
    if (GROUPED && corr.gcols <= 0) return hipErrorInvalidValue;
    const int per_cu = ls.per_cu.load(std::memory_order_relaxed);
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int ntiles = tiles_m * tiles_n;
    const int per_xcd = (ntiles + 7) / 8;
    // one resident workgroup per slot: 32 CUs per XCD on gfx950 (256 in all)
    const int nslots = std::min(per_xcd, 32 * per_cu);
    hipLaunchKernelGGL(kfn, dim3((unsigned)(8 * nslots)), dim3(64 * WM * WN), smem, st, A, lda, B, ldb, M, N, K,
                       tiles_n, ntiles, per_xcd, corr, epi);
    return hipGetLastError();
}

// Tile shape with the smallest estimated time: rounds of 256 concurrent tiles
// times tile area, with smaller tiles charged for their higher LDS and L2
// traffic per MFMA (weights from timings of the shapes on gfx950).
enum class Shape { T256x256, T256x160, T256x128, T128x128, T64x64 };

// gcols > 0: only shapes whose tile width divides gcols (a tile must not
// straddle two groups of a grouped A operand).
bool pick_shape(int64_t M, int64_t N, int gcols, Shape &best) {
    best = Shape::T64x64;
    const bool fits64 = gcols <= 0 || gcols % 64 == 0;
    if (N <= 64) return fits64;
    // 64 x 64 tiles only win where the whole product is a round or less of
    // them (a single instance of a few hundred tokens): there a large tile
    // leaves all but a few CUs idle and its K loop is the whole time
    struct C { Shape s; int bm, bn; double w; } cands[] = {
        {Shape::T256x256, 256, 256, 1.0}, {Shape::T256x160, 256, 160, 1.2}, {Shape::T256x128, 256, 128, 1.16},
        {Shape::T128x128, 128, 128, 1.3}, {Shape::T64x64, 64, 64, 2.5}};
    best = Shape::T128x128;
    double best_cost = 1e300;
    bool found = false;
    for (const C &c : cands) {
        if (gcols > 0 && gcols % c.bn != 0) continue;
        const double tiles = (double)((M + c.bm - 1) / c.bm) * (double)((N + c.bn - 1) / c.bn);
        const double rounds = std::ceil(tiles / 256.0);
        const double cost = rounds * c.bm * c.bn * c.w;
        if (cost < best_cost) {
            best_cost = cost;
            best = c.s;
            found = true;
        }
    }
    if (!found) best = Shape::T64x64;
    return found || fits64;
}

template <typename E, bool ROWS, bool CORR, bool GROUPED, class Epi>
hipError_t launch_shape(Shape shape, const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N,
                        int64_t K, const Corr<E> &corr, Epi epi, hipStream_t st, bool setup_only) {
    switch (shape) {
    case Shape::T256x256:
        // float32 keeps 64-byte slices (128 would spill it)
        if constexpr (sizeof(E) == 4)
            return gemm_launch<E, 256, 256, 4, 2, 4, 64, ROWS, CORR, GROUPED>(A, lda, B, ldb, M, N, K, corr, epi, st,
                                                                              setup_only);
        else return gemm_launch<E, 256, 256, 4, 2, 2, 128, ROWS, CORR, GROUPED>(A, lda, B, ldb, M, N, K, corr, epi, st,
                                                                               setup_only);
    case Shape::T256x160:
        return gemm_launch<E, 256, 160, 8, 1, 3, 128, ROWS, CORR, GROUPED>(A, lda, B, ldb, M, N, K, corr, epi, st,
                                                                           setup_only);
    case Shape::T256x128:
        return gemm_launch<E, 256, 128, 4, 2, 3, 128, ROWS, CORR, GROUPED>(A, lda, B, ldb, M, N, K, corr, epi, st,
                                                                           setup_only);
    case Shape::T128x128:
        return gemm_launch<E, 128, 128, 2, 2, 4, 128, ROWS, CORR, GROUPED>(A, lda, B, ldb, M, N, K, corr, epi, st,
                                                                           setup_only);
    case Shape::T64x64:
        return gemm_launch<E, 64, 64, 2, 2, 4, 128, ROWS, CORR, GROUPED>(A, lda, B, ldb, M, N, K, corr, epi, st,
                                                                         setup_only);
    }
    return hipErrorInvalidValue;
}

// Float32 products of only a few tiles (a single instance of a few hundred
// tokens).  There a 64 x 64 tile's wavefronts each run the whole contraction
// through one chain of v_mfma_f32_32x32x2f32 (64 cycles each, K / 2 of them),
// so the product takes that chain's time on a handful of CUs.  Here a
// workgroup owns one 32 x 32 block and its four wavefronts split the 16-deep
// steps between them (step s to wavefront s % 4); their partial blocks meet in
// LDS and wavefront 0 applies the epilogue.  Operands are read straight from
// global memory in fragment form, kSmallGroup steps requested at once.
// With CORR the output product's correction steps follow the static ones as
// in gemm_kernel: for each instance b with rows in the block, kc / 16 steps of
// A's correction columns (rows of other instances zeroed) against R1_b.
constexpr int kSmallWaves = 4;
constexpr int kSmallGroup = 3;

template <bool ROWS, bool CORR, class Epi>
__global__ __launch_bounds__(64 * kSmallWaves) void small_gemm_f32_kernel(const float *__restrict__ A, int64_t lda,
                                                                          const float *__restrict__ B, int64_t ldb,
                                                                          int64_t M, int64_t N, int64_t K,
                                                                          Corr<float> corr, Epi epi) {
    __shared__ float red[kSmallWaves - 1][16][64];  // partial blocks of wavefronts 1..3, [register][lane]
    __shared__ __align__(16) float cts[32];         // the block's per-column terms
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, hf = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.y * 32, col0 = (int64_t)blockIdx.x * 32;
    // rows past M or N are read from the last row and never stored
    const int64_t ra = row0 + lr < M ? row0 + lr : M - 1, rb = col0 + lr < N ? col0 + lr : N - 1;
    const float *pa = A + ra * lda + 8 * hf, *pb = B + rb * ldb + 8 * hf;
    bool has_ct = false;
    if constexpr (Epi::kColumnTerms) {
        has_ct = epi.bias != nullptr;
        if (has_ct && tid < 32) cts[tid] = col0 + tid < epi.ncols ? to_f32(epi.bias[col0 + tid]) : 0.f;
    }
    const int S0 = (int)(K / 16);
    int S = S0, SC = 1;
    int64_t b_first = 0;
    if constexpr (CORR) {
        const int64_t rend = row0 + 32 < M ? row0 + 32 : M;
        b_first = row0 / corr.n;
        SC = corr.kc / 16;
        S = S0 + (int)((rend - 1) / corr.n - b_first + 1) * SC;
    }
    f32x16 acc = f32x16{};
    for (int s0 = wave; s0 < S; s0 += kSmallWaves * kSmallGroup) {
        f32x8 fa[kSmallGroup], fb[kSmallGroup];
#pragma unroll
        for (int u = 0; u < kSmallGroup; ++u) {
            const int s = s0 + kSmallWaves * u;
            const int sl = s < S ? s : s0;  // a step past the end re-reads s0 and is skipped
            if (!CORR || sl < S0) {
                fa[u] = ld_frag(pa + 16 * (int64_t)sl);
                fb[u] = ld_frag(pb + 16 * (int64_t)sl);
            } else {
                const int q = sl - S0, j = q % SC;
                const int64_t b = b_first + q / SC;
                const int64_t kk = 16 * (int64_t)j + 8 * hf;
                fa[u] = ld_frag(A + ra * lda + corr.kcol + kk);
                const int64_t r = row0 + lr;
                if (!(r >= b * corr.n && r < (b + 1) * corr.n)) fa[u] = f32x8{};
                fb[u] = ld_frag(corr.R1t + b * corr.rstride + rb * corr.kc + kk);
            }
        }
#pragma unroll
        for (int u = 0; u < kSmallGroup; ++u)
            if (s0 + kSmallWaves * u < S) acc = ROWS ? mma16(acc, fb[u], fa[u]) : mma16(acc, fa[u], fb[u]);
    }
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t) red[wave - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kSmallWaves - 1; ++w)
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] += red[w][t][lane];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float v[4] = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        const int64_t r = ROWS ? row0 + lr : row0 + acc_row(lane, 4 * g);
        const int64_t c = ROWS ? col0 + acc_row(lane, 4 * g) : col0 + lr;
        epi.fix4(v, r, c, has_ct ? cts + (c - col0) : nullptr);
        if (r < M && c < N) epi.store4(r, c, pack4<float>(v));
    }
}

// The 64 x 64 tiles of a product that leaves most CUs idle take the small
// kernel instead (float32 only: a 16-deep bf16 step is one MFMA where float32
// needs eight).
constexpr int64_t kSmallMaxTiles = 32;

template <typename E, bool ROWS, bool CORR, bool GROUPED = false, class Epi>
hipError_t gemm_dispatch(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                         const Corr<E> &corr, Epi epi, hipStream_t st) {
    if constexpr (sizeof(E) == 4 && !GROUPED) {
        if (((M + 63) / 64) * ((N + 63) / 64) <= kSmallMaxTiles) {
            if (K % 16 != 0 || (CORR && (corr.n < 1 || corr.kc < 16 || corr.kc % 16 != 0)))
                return hipErrorInvalidValue;
            hipLaunchKernelGGL((small_gemm_f32_kernel<ROWS, CORR, Epi>),
                               dim3((unsigned)((N + 31) / 32), (unsigned)((M + 31) / 32)), dim3(64 * kSmallWaves), 0,
                               st, A, lda, B, ldb, M, N, K, corr, epi);
            return hipGetLastError();
        }
    }
    Shape shape;
    if (!pick_shape(M, N, GROUPED ? corr.gcols : 0, shape)) return hipErrorInvalidValue;
    return launch_shape<E, ROWS, CORR, GROUPED>(shape, A, lda, B, ldb, M, N, K, corr, epi, st, false);
}

// The one-time set-up of every tile shape of one kernel family.
template <typename E, bool ROWS, bool CORR, bool GROUPED, class Epi> hipError_t setup_family() {
    for (Shape sh : {Shape::T256x256, Shape::T256x160, Shape::T256x128, Shape::T128x128, Shape::T64x64}) {
        const hipError_t e = launch_shape<E, ROWS, CORR, GROUPED>(sh, nullptr, 0, nullptr, 0, 0, 0, 0, Corr<E>{},
                                                                  Epi{}, nullptr, true);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

template <typename E> hipError_t gemm_prepare() {
    hipError_t e;
    if ((e = setup_family<E, true, false, false, RowStore<E>>()) != hipSuccess) return e;   // left pass, dense
    if ((e = setup_family<E, true, false, true, RowStore<E>>()) != hipSuccess) return e;    // grouped (BLAST)
    if ((e = setup_family<E, false, false, false, R1tStore<E>>()) != hipSuccess) return e;  // right factor
    if ((e = setup_family<E, true, true, false, RowStore<E>>()) != hipSuccess) return e;    // output
    return setup_family<E, true, true, true, RowStore<E>>();                                // BLAST output
}

template <typename E>
hipError_t launch_gemm_store(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                             E *D, int64_t ldd, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    return gemm_dispatch<E, true, false>(A, lda, B, ldb, M, N, K, Corr<E>{}, RowStore<E>{D, ldd}, st);
}

bool gemm_groupable(int64_t M, int64_t N, int gcols) {
    Shape shape;
    return gcols > 0 && N % gcols == 0 && pick_shape(M, N, gcols, shape);
}

template <typename E>
hipError_t launch_gemm_store_grouped(const E *A, int64_t lda, const E *B, int64_t ldb, int64_t M, int64_t N,
                                     int64_t K, int gcols, int64_t gstride, E *D, int64_t ldd, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (gcols <= 0 || N % gcols != 0) return hipErrorInvalidValue;
    Corr<E> g{};
    g.gcols = gcols;
    g.gstride = gstride;
    return gemm_dispatch<E, true, false, true>(A, lda, B, ldb, M, N, K, g, RowStore<E>{D, ldd}, st);
}

template <typename E>
hipError_t launch_right(const E *Mp, const E *Wres_t, int64_t rows, int64_t c1, int64_t c2, int kc, float alpha,
                        E *R1t, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    return gemm_dispatch<E, false, false>(Mp, c1, Wres_t, c1, rows, c2, c1, Corr<E>{},
                                          R1tStore<E>{R1t, kc, c2, alpha}, st);
}

template <typename E>
hipError_t launch_output_ex(const E *A, int64_t lda, int64_t K, const E *B, int64_t ldb, int kcol, int kc,
                            const E *R1t, int64_t rstride, int64_t Ntok, int64_t n, int64_t N, const E *bias, E *Y,
                            int64_t ldy, int gcols, int64_t gstride, hipStream_t st) {
    if (Ntok <= 0) return hipSuccess;
    if (kc > 0 && (n < 1 || kc > 256 || kc % 16 != 0)) return hipErrorInvalidValue;
    if (gcols < 0 || (gcols > 0 && N % gcols != 0)) return hipErrorInvalidValue;
    const RowStore<E> epi{Y, ldy, bias, N};
    Corr<E> c{R1t, n, kcol, kc, rstride, gcols, gstride};
    if (kc == 0) {
        c.R1t = nullptr;
        if (gcols > 0) return gemm_dispatch<E, true, false, true>(A, lda, B, ldb, Ntok, N, K, c, epi, st);
        return gemm_dispatch<E, true, false>(A, lda, B, ldb, Ntok, N, K, c, epi, st);
    }
    if (gcols > 0) return gemm_dispatch<E, true, true, true>(A, lda, B, ldb, Ntok, N, K, c, epi, st);
    return gemm_dispatch<E, true, true>(A, lda, B, ldb, Ntok, N, K, c, epi, st);
}

template <typename E>
hipError_t launch_output(const E *T, int64_t ldt, int kw, int kc, const E *Vs, const E *R1t, int64_t Ntok,
                         int64_t n, int64_t c2, const E *bias, E *Y, hipStream_t st) {
    return launch_output_ex<E>(T, ldt, kw, Vs, kw, kw, kc, R1t, c2 * kc, Ntok, n, c2, bias, Y, c2, 0, 0, st);
}

template hipError_t gemm_prepare<bf16>();
template hipError_t gemm_prepare<float>();
template hipError_t launch_gemm_store<bf16>(const bf16 *, int64_t, const bf16 *, int64_t, int64_t, int64_t, int64_t,
                                            bf16 *, int64_t, hipStream_t);
template hipError_t launch_gemm_store<float>(const float *, int64_t, const float *, int64_t, int64_t, int64_t,
                                             int64_t, float *, int64_t, hipStream_t);
template hipError_t launch_right<bf16>(const bf16 *, const bf16 *, int64_t, int64_t, int64_t, int, float, bf16 *,
                                       hipStream_t);
template hipError_t launch_right<float>(const float *, const float *, int64_t, int64_t, int64_t, int, float, float *,
                                        hipStream_t);
template hipError_t launch_output_ex<bf16>(const bf16 *, int64_t, int64_t, const bf16 *, int64_t, int, int,
                                           const bf16 *, int64_t, int64_t, int64_t, int64_t, const bf16 *, bf16 *,
                                           int64_t, int, int64_t, hipStream_t);
template hipError_t launch_output_ex<float>(const float *, int64_t, int64_t, const float *, int64_t, int, int,
                                            const float *, int64_t, int64_t, int64_t, int64_t, const float *,
                                            float *, int64_t, int, int64_t, hipStream_t);
template hipError_t launch_gemm_store_grouped<bf16>(const bf16 *, int64_t, const bf16 *, int64_t, int64_t, int64_t,
                                                    int64_t, int, int64_t, bf16 *, int64_t, hipStream_t);
template hipError_t launch_gemm_store_grouped<float>(const float *, int64_t, const float *, int64_t, int64_t,
                                                     int64_t, int64_t, int, int64_t, float *, int64_t, hipStream_t);
template hipError_t launch_output<bf16>(const bf16 *, int64_t, int, int, const bf16 *, const bf16 *, int64_t,
                                        int64_t, int64_t, const bf16 *, bf16 *, hipStream_t);
template hipError_t launch_output<float>(const float *, int64_t, int, int, const float *, const float *, int64_t,
                                         int64_t, int64_t, const float *, float *, hipStream_t);

}  // namespace dyra
