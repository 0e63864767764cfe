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
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
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

// One sequence of a call as the scan kernels see it: a sequence of the batch,
// or one document of a packed stream (the fast weight restarts from W_down0
// at every document start). Its tokens are rows xrow0 .. xrow0+len-1 of x and
// y; the target of position t is ids[id0 + t + 1]; its scratch slots start at
// slot0 (a multiple of 256) and its snapshot groups at grp0. It starts from
// state state_in (-1: zero, i.e. W_down0) and leaves its final state in
// state_out of the output state buffer (-1: nowhere).
struct SeqInfo {
  long long xrow0, id0;
  int slot0, len, grp0, state_in, state_out, pad_;
};

// The sequences of a call. Without a table (info null) they are the B
// sequences of T tokens of a batch: sequence b has rows b*T.., ids from
// b*(T+1), slots b*T_pad.., groups b*ngroups.., and its own state b in and out.
// With a table, tile_seq maps each 256-slot tile and group_seq each group to
// its sequence (device arrays).
struct Seqs {
  const SeqInfo *info;
  const int *tile_seq;
  const int *group_seq;
  int T, T_pad, ngroups;
  __device__ __forceinline__ SeqInfo at(int j) const {
    if (info) return info[j];
    SeqInfo s;
    s.xrow0 = (long long)j * T;
    s.id0 = (long long)j * (T + 1);
    s.slot0 = j * T_pad;
    s.len = T;
    s.grp0 = j * ngroups;
    s.state_in = j;
    s.state_out = j;
    s.pad_ = 0;
    return s;
  }
  __device__ __forceinline__ int of_tile(int tile) const { return info ? tile_seq[tile] : tile / (T_pad / 256); }
  __device__ __forceinline__ int of_group(int g) const { return info ? group_seq[g] : g / ngroups; }
};

// The positions of one call: tokens 0..T-1 of each sequence, grouped in
// chunks of C and snapshot groups of L = G*C tokens; scratch buffers hold
// T_pad >= T slots per sequence, zero beyond T.
// With a sequence table (packed documents, bf16 path): nseq sequences of their
// own lengths, S scratch slots and G groups in total, each sequence padded to
// a multiple of 256 slots; B, T, T_pad and ngroups then describe the
// caller's arrays only (x, y: [B][T][d]; ids: [B][T+1]).
struct Layout {
  int B, T, T_pad, C, L, ngroups, d, f;
  int intra;  // 1 when a group holds more than one chunk
  bool tab = false;  // sequences from a table (info, tile_seq, group_seq: device arrays)
  const SeqInfo *info = nullptr;
  const int *tile_seq = nullptr, *group_seq = nullptr;
  int nseq = 0, S = 0, G = 0;
  // sequences, scratch slots and groups in total
  int n_seq() const { return tab ? nseq : B; }
  long long n_slots() const { return tab ? (long long)S : (long long)B * T_pad; }
  long long n_groups() const { return tab ? (long long)G : (long long)B * ngroups; }
  Seqs seqs() const { return Seqs{info, tile_seq, group_seq, T, T_pad, ngroups}; }
};

static inline long long round_up_ll(long long a, long long b) { return (a + b - 1) / b * b; }
