// MFMA building blocks for gfx950 (CDNA4), shared by the libdyra kernels.
//
// Operand fragments: for a 32x32 output block and a 16-deep slice of the
// contraction, lane l (0..63) of a wavefront holds 8 consecutive contraction
// elements k = 8*(l/32) .. 8*(l/32)+7 of row (A) or column (B) l%32.  For bf16
// that is one v_mfma_f32_32x32x16_bf16.  For float32 the same 8 elements feed
// eight v_mfma_f32_32x32x2_f32 steps: step t contracts k = t (lanes 0-31) and
// k = 8+t (lanes 32-63), so A and B use one and the same permutation of k and
// the sum is unchanged.
//
// Accumulator layout (both instructions): lane l holds column l%32 and, in
// register t, row 8*(t/4) + 4*(l/32) + (t%4) of the 32x32 block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dyra {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16 raw bytes (a struct vector type such as uint4 in an array stays in scratch)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename E> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

// Elements per 16-byte vector and LDS row padding (elements) that keeps
// ds_read_b128 row accesses on distinct banks.
template <typename E> struct Lay {
    static constexpr int VEC = 16 / (int)sizeof(E);
    static constexpr int PAD = 16 / (int)sizeof(E);
};

__device__ __forceinline__ f32x16 mma16(f32x16 acc, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mma16(f32x16 acc, f32x8 a, f32x8 b) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], acc, 0, 0, 0);
    return acc;
}

// Fragment at `p` (8 consecutive elements, 16-byte aligned).
__device__ __forceinline__ bf16x8 ld_frag(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f32x8 ld_frag(const float *p) {
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(p + 4);
    f32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

__device__ __forceinline__ bf16x8 zero_frag(const bf16x8 &) { return bf16x8{}; }
__device__ __forceinline__ f32x8 zero_frag(const f32x8 &) { return f32x8{}; }

template <typename E> __device__ __forceinline__ E to_elem(float v);
template <> __device__ __forceinline__ bf16 to_elem<bf16>(float v) { return static_cast<bf16>(v); }
template <> __device__ __forceinline__ float to_elem<float>(float v) { return v; }

__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// Row of the accumulator register t for lane l (see the layout note above).
__device__ __forceinline__ int acc_row(int lane, int t) { return 8 * (t >> 2) + 4 * (lane >> 5) + (t & 3); }

// Asynchronous 16-byte copy global -> LDS (global_load_lds_dwordx4): lane l
// writes LDS bytes [lds + 16 l, lds + 16 l + 16); lds must be wave-uniform.
// Completion is tracked by the vector-memory counter only.
__device__ __forceinline__ void lds_dma16(const void *g, char *lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that the compiler may not move memory accesses across and
// that adds no wait of its own (the waits are explicit).
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace dyra
