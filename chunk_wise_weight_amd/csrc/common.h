// Shared device-side types and helpers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float x) { return __builtin_bit_cast(bf16_t, (__bf16)x); }

// Non-temporal stores (the `nt` bit): for results no later instruction of
// the same kernel reads, so that they do not push the operand tiles other
// workgroups are still reading out of L2.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt(void *p, uint32_t lo, uint32_t hi) {
  __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t *>(p));
}
__device__ __forceinline__ void store_nt(bf16_t *p, bf16_t v) { __builtin_nontemporal_store(v, p); }

// SiLU(g) = g / (1 + e^-g) in fp32 with the hardware reciprocal (v_rcp_f32,
// within 1 ulp) in place of an IEEE division: within a few fp32 ulp of the
// division form, far below the bf16 rounding of the values it feeds, at a
// third of the instructions.
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// One K-segment of a GEMM operand: row r, column k (segment-local) lives at
// base[r * ld + k]. Rows >= nrows and columns >= kvalid read as zero.
template <typename T>
struct Seg {
  const T *base;
  long long ld;
  int nrows;
  int kvalid;
};

// The positions of one call: tokens 0..T-1 of each sequence, grouped in
// chunks of C and snapshot groups of L = G*C tokens; scratch buffers hold
// T_pad >= T slots per sequence, zero beyond T.
struct Layout {
  int B, T, T_pad, C, L, ngroups, d, f;
  int intra;  // 1 when a group holds more than one chunk
};

static inline long long round_up_ll(long long a, long long b) { return (a + b - 1) / b * b; }
