// bf16 MFMA kernels of the chunk-wise fast-weight path (gfx950).
//
// Every contraction is written as D[i][j] = sum_k A[i][k] * B[j][k] with both
// operands K-contiguous ("NT" form). A block computes a 256 x 256 tile with 4
// waves (2 x 2), each wave 128 x 128 as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16
// with fp32 accumulators (256 AGPRs per lane).
//
// K advances in stages of 32 through a ring of 4 LDS stages (32 KB each, 128
// KB in all): while a stage is multiplied, the next three are in flight. Tiles
// go from HBM straight into LDS with 16-byte buffer loads (no register
// staging); each wave waits only for the oldest stage it needs. The four
// 16-byte chunks of each 64-byte LDS row are XOR-swizzled so that the MFMA
// fragment reads are free of bank conflicts. Rows or columns outside an
// operand's valid range are fetched through an out-of-range buffer offset,
// which the hardware returns as zero.
//
// Operands are either row-major (element (r, k) at r*ld + k) or K-blocked by
// 64 (element (r, k) at (k/64)*kblk + r*64 + k%64): the token-indexed operands
// of the update (eta Z^T and V^T) are stored K-blocked so that one stage reads
// one contiguous slab instead of 256 rows strided by the whole stream length.
//
// MFMA 32x32x16 register layout (lane l, accumulator register r):
//   A operand: row i = l % 32, k = 8*(l/32) .. +7;  B operand: column j = l % 32, same k.
//   D: j = l % 32, i = 8*(r/4) + 4*(l/32) + r%4.
// So each lane holds, per group of 4 registers, four consecutive i for one j:
// epilogues store 4 consecutive elements along i.
#include "launch.h"

namespace {

constexpr int BM = 256;  // tile rows along i
constexpr int BN = 256;  // tile rows along j
constexpr int BK = 32;   // k per stage
constexpr int NS = 4;    // stages in the LDS ring
constexpr int NTHREADS = 256;
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer descriptor word 3 on the gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;   // offset past num_records: the load returns zero

struct Acc {
  f32x16 v[4][4];
};

typedef __attribute__((address_space(3))) void lds_void;
typedef bf16_t Stage[2][BM * BK];  // [operand A/B][256 rows x 32]

// One K-segment of an operand, rows [0, nrows) valid, columns [0, kvalid) valid.
struct Opnd {
  const bf16_t *base;
  long long ld;    // row-major: row pitch in elements
  long long kblk;  // K-blocked: elements per 64-column block (0 = row-major)
  int nrows;
  int kvalid;
  int koff;        // K-blocked: absolute column of segment column 0
};

__device__ __forceinline__ Opnd rowmajor(const bf16_t *base, long long ld, int nrows, int kvalid) {
  return Opnd{base, ld, 0, nrows, kvalid, 0};
}
__device__ __forceinline__ Opnd kblocked(const bf16_t *base, long long kblk, int nrows, int kvalid, int koff) {
  return Opnd{base, 64, kblk, nrows, kvalid, koff};
}

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
// element offset of (row r, 16-byte chunk c) inside a 256 x 32 bf16 LDS tile
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }

__device__ __forceinline__ void acc_zero(Acc &acc) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.v[bi][bj][r] = 0.f;
}

// Queue the copy of rows [row0, row0+256) x cols [k, k+32) of one operand into
// an LDS tile. Wave w moves rows w*64 .. w*64+63, sixteen rows per
// instruction; lane l of an instruction fills row r0 + l/4, physical chunk
// l%4, so it fetches the logical chunk (l%4) ^ swz(row). One descriptor per
// call; each instruction's row offset goes in soffset.
template <bool BLOCKED>
__device__ __forceinline__ void issue_tile(bf16_t *lds_tile, const Opnd &s, int row0, int k, int w, int lane) {
  const int lr = lane >> 2;
  const int nvw = s.nrows - row0 - w * 64;  // valid rows among this wave's 64
  if (!BLOCKED) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(s.base + (long long)row0 * s.ld + k), (short)0, 0x7fffffff, kBufferFlags);
    const int ldb = (int)s.ld * 2;
    const int kleft = s.kvalid - k;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int slab = w * 64 + n * 16;
      const int c = (lane & 3) ^ swz(slab + lr);
      const bool ok = (n * 16 + lr) < nvw && c * 8 < kleft;
      const uint32_t voff = ok ? (uint32_t)(lr * ldb + c * 16) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lds_tile + slab * BK), 16, voff, slab * ldb, 0, 0);
    }
  } else {
    const int ka0 = s.koff + k;  // absolute column of this stage's first column
    const int kb0 = ka0 >> 6;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(s.base + (long long)kb0 * s.kblk + (long long)row0 * 64), (short)0, 0x7fffffff,
        kBufferFlags);
    const int blkb = (int)s.kblk * 2;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int slab = w * 64 + n * 16;
      const int c = (lane & 3) ^ swz(slab + lr);
      const int ka = ka0 + c * 8;
      const bool ok = (n * 16 + lr) < nvw && (k + c * 8) < s.kvalid;
      const uint32_t voff =
          ok ? (uint32_t)(((ka >> 6) - kb0) * blkb + lr * 128 + (ka & 63) * 2) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lds_tile + slab * BK), 16, voff, slab * 128, 0, 0);
    }
  }
}

template <bool ABLK, bool BBLK>
__device__ __forceinline__ void issue_stage(Stage &st, const Opnd &a, const Opnd &b, int arow0, int brow0, int k,
                                            int w, int lane) {
  issue_tile<ABLK>(st[0], a, arow0, k, w, lane);
  issue_tile<BBLK>(st[1], b, brow0, k, w, lane);
}

// Wait until at most `later` stages of this wave's loads (8 loads per stage)
// are still in flight, then for every wave: their loads of the awaited stage
// have landed too, and every wave is done with the stage computed before.
__device__ __forceinline__ void stage_wait(int later) {
  if (later >= 2)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (later == 1)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// One 32-deep stage: 2 k-substeps of 16, 16 MFMAs each.
__device__ __forceinline__ void mma_stage(Acc &acc, const bf16_t *lA, const bf16_t *lB, int wm, int wn, int lane) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = 2 * ks + (lane >> 5);
    bf16x8 a[4], b[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
      a[bi] = *reinterpret_cast<const bf16x8 *>(lA + lds_off(wm * 128 + bi * 32 + (lane & 31), c));
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
      b[bj] = *reinterpret_cast<const bf16x8 *>(lB + lds_off(wn * 128 + bj * 32 + (lane & 31), c));
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
        acc.v[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc.v[bi][bj], 0, 0, 0);
  }
}

// K loop over segment 1 (nk1 stages, both operands row-major) then segment 2
// (nk2 stages; its A operand K-blocked when A2BLK).
template <bool A2BLK>
__device__ __forceinline__ void gemm_loop(Acc &acc, Stage *ring, const Opnd &a1, const Opnd &b1, int nk1,
                                          const Opnd &a2, const Opnd &b2, int nk2, int arow0, int brow0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1, wn = w & 1;
  const int nk = nk1 + nk2;
  auto issue = [&](int kt) {
    if (kt < nk1)
      issue_stage<false, false>(ring[kt % NS], a1, b1, arow0, brow0, kt * BK, w, lane);
    else
      issue_stage<A2BLK, false>(ring[kt % NS], a2, b2, arow0, brow0, (kt - nk1) * BK, w, lane);
  };
  for (int kt = 0; kt < NS - 1 && kt < nk; ++kt) issue(kt);
  for (int kt = 0; kt < nk; ++kt) {
    const int later = (nk - 1 - kt) < (NS - 2) ? (nk - 1 - kt) : (NS - 2);
    stage_wait(later);
    if (kt + NS - 1 < nk) issue(kt + NS - 1);
    mma_stage(acc, ring[kt % NS][0], ring[kt % NS][1], wm, wn, lane);
  }
}

// ---------------------------------------------------------------------------
// Up/gate GEMM with SwiGLU epilogue. i = token slot, j = interleaved W_ug row.
// Writes Z [B][T_pad][f] (row-major) and eta*Z^T K-blocked [B][T_pad/64][f][64].
// grid: (2f/256, B*T_pad/256)
struct A1Args {
  const bf16_t *x;
  const bf16_t *Wug;
  bf16_t *Z;
  bf16_t *ZT;
  float eta;
  int write_zt;
  int T, T_pad, d, f;
};

__global__ __launch_bounds__(NTHREADS, 1) void k_a1(A1Args p) {
  __shared__ __attribute__((aligned(16))) Stage ring[NS];
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int b = m0 / p.T_pad;
  const int pos0 = m0 - b * p.T_pad;
  const Opnd sa = rowmajor(p.x + ((long long)b * p.T + pos0) * p.d, p.d, p.T - pos0, p.d);
  const Opnd sb = rowmajor(p.Wug + (long long)n0 * p.d, p.d, 2 * p.f - n0, p.d);
  Acc acc;
  acc_zero(acc);
  gemm_loop<false>(acc, ring, sa, sb, p.d / BK, sa, sb, 0, 0, 0);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  bf16_t *ZTb = p.ZT + (long long)b * p.f * p.T_pad;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int feat = (n0 + wn * 128) / 2 + pr * 32 + (lane & 31);
      if (feat >= p.f) continue;
      const f32x16 &u = acc.v[bi][2 * pr];
      const f32x16 &g = acc.v[bi][2 * pr + 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pos = pos0 + wm * 128 + bi * 32 + 8 * q + 4 * (lane >> 5);
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = silu_f32(g[4 * q + r]) * u[4 * q + r];
        if (p.write_zt) {
          uint2 pk;
          pk.x = pack_bf16x2(p.eta * z[0], p.eta * z[1]);
          pk.y = pack_bf16x2(p.eta * z[2], p.eta * z[3]);
          *reinterpret_cast<uint2 *>(ZTb + ((long long)(pos >> 6) * p.f + feat) * 64 + (pos & 63)) = pk;
        }
        bf16_t *zrow = p.Z + ((long long)b * p.T_pad + pos) * p.f + feat;
#pragma unroll
        for (int r = 0; r < 4; ++r) zrow[(long long)r * p.f] = f32_to_bf16(z[r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// State update with snapshots. i = hidden unit (ZT row), j = model dim (VT row),
// k = token slot. The fp32 accumulators ARE the state W[a][i] for the tile and
// stay in registers for the whole token stream; at each group start g*L the
// tile is written out as a bf16 snapshot.
// grid: (f/256, d/256, B)
struct UpdArgs {
  const bf16_t *ZT;
  const bf16_t *VT;
  float *state;
  bf16_t *snap;
  int T_pad, kend, L, ngroups, d, f;
};

// Write the accumulator tile as bf16 into a snapshot W[a][i] ([d][f]).
// `lane_ptr` points at this lane's first element (a = j0 + wn*128 + l%32,
// i = i0 + wm*128 + 4*(l/32)); tiles are always full (d, f multiples of 256).
__device__ __forceinline__ void dump_snapshot(const Acc &acc, bf16_t *lane_ptr, int f) {
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    bf16_t *row = lane_ptr + (long long)bj * 32 * f;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 pk;
        pk.x = pack_bf16x2(acc.v[bi][bj][4 * q + 0], acc.v[bi][bj][4 * q + 1]);
        pk.y = pack_bf16x2(acc.v[bi][bj][4 * q + 2], acc.v[bi][bj][4 * q + 3]);
        *reinterpret_cast<uint2 *>(row + bi * 32 + 8 * q) = pk;
      }
    __builtin_amdgcn_sched_barrier(0);  // one column block at a time: bounded register use
  }
}

__global__ __launch_bounds__(NTHREADS, 1) void k_update(UpdArgs p) {
  __shared__ __attribute__((aligned(16))) Stage ring[NS];
  const int i0 = blockIdx.x * BM;
  const int j0 = blockIdx.y * BN;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1, wn = w & 1;
  const long long df = (long long)p.d * p.f;
  // this lane's first element of the tile, relative to W[0][0]
  const long long lane_off =
      (long long)(j0 + wn * 128 + (lane & 31)) * p.f + i0 + wm * 128 + 4 * (lane >> 5);
  float *st = p.state + b * df + lane_off;
  bf16_t *snap0 = p.snap + (long long)b * p.ngroups * df + lane_off;

  Acc acc;
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const float *row = st + (long long)bj * 32 * p.f;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(row + bi * 32 + 8 * q);
        acc.v[bi][bj][4 * q + 0] = v.x;
        acc.v[bi][bj][4 * q + 1] = v.y;
        acc.v[bi][bj][4 * q + 2] = v.z;
        acc.v[bi][bj][4 * q + 3] = v.w;
      }
  }

  const Opnd sa = kblocked(p.ZT + (long long)b * p.f * p.T_pad, (long long)p.f * 64, p.f, p.T_pad, 0);
  const Opnd sb = kblocked(p.VT + (long long)b * p.d * p.T_pad, (long long)p.d * 64, p.d, p.T_pad, 0);
  const int nk = p.kend / BK;
  for (int kt = 0; kt < NS - 1 && kt < nk; ++kt)
    issue_stage<true, true>(ring[kt % NS], sa, sb, i0, j0, kt * BK, w, lane);
  // Group starts are multiples of the stage depth: snapshot g is written
  // between stages, while the following stages are already in flight.
  int kt = 0;
  for (int g = 0; g < p.ngroups; ++g) {
    dump_snapshot(acc, snap0 + (long long)g * df, p.f);
    const int kt_end = (g + 1 < p.ngroups) ? (g + 1) * (p.L / BK) : nk;
    for (; kt < kt_end; ++kt) {
      const int later = (nk - 1 - kt) < (NS - 2) ? (nk - 1 - kt) : (NS - 2);
      stage_wait(later);
      if (kt + NS - 1 < nk)
        issue_stage<true, true>(ring[(kt + NS - 1) % NS], sa, sb, i0, j0, (kt + NS - 1) * BK, w, lane);
      mma_stage(acc, ring[kt % NS][0], ring[kt % NS][1], wm, wn, lane);
    }
  }
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    float *row = st + (long long)bj * 32 * p.f;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(row + bi * 32 + 8 * q) =
            make_float4(acc.v[bi][bj][4 * q + 0], acc.v[bi][bj][4 * q + 1], acc.v[bi][bj][4 * q + 2],
                        acc.v[bi][bj][4 * q + 3]);
  }
}

// ---------------------------------------------------------------------------
// Within-group scores P[t][s] = eta <z_t, z_s> for s in an earlier chunk of the
// same group. i = s, j = t; only tiles with i-tile <= j-tile are formed.
// grid: (nt*nt, ngroups, B), nt = ceil(L/256)
struct ScoreArgs {
  const bf16_t *Z;
  bf16_t *P;
  float eta;
  int T, T_pad, L, C, ngroups, f, nt;
};

__global__ __launch_bounds__(NTHREADS, 1) void k_scores(ScoreArgs p) {
  __shared__ __attribute__((aligned(16))) Stage ring[NS];
  const int it = blockIdx.x % p.nt, jt = blockIdx.x / p.nt;
  const int g = blockIdx.y, b = blockIdx.z;
  const long long gs = (long long)g * p.L;
  const int Lg = (int)((p.T - gs) < p.L ? (p.T - gs) : p.L);
  const int i0 = it * BM, j0 = jt * BN;
  if (it > jt || j0 >= Lg) return;
  const Opnd s = rowmajor(p.Z + ((long long)b * p.T_pad + gs) * p.f, p.f, (int)(p.T_pad - gs), p.f);
  Acc acc;
  acc_zero(acc);
  gemm_loop<false>(acc, ring, s, s, p.f / BK, s, s, 0, i0, j0);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  bf16_t *Pg = p.P + ((long long)b * p.ngroups + g) * p.L * p.L;
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const int t = j0 + wn * 128 + bj * 32 + (lane & 31);
    if (t >= p.L) continue;
    const int ct = t / p.C;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int sidx = i0 + wm * 128 + bi * 32 + 8 * q + 4 * (lane >> 5);
        if (sidx >= p.L) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = ((sidx + r) / p.C < ct) ? p.eta * acc.v[bi][bj][4 * q + r] : 0.f;
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(Pg + (long long)t * p.L + sidx) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// Output GEMM: y[gL+t][a] = sum_k [snap | V^T][a][k] * [Z | P][t][k].
// i = a (model dim), j = t (token within group).
// grid: (d/256, ceil(L/256), B*ngroups)
struct OutArgs {
  const bf16_t *Z;
  const bf16_t *P;
  const bf16_t *snap;
  const bf16_t *VT;
  bf16_t *y;
  int T, T_pad, L, C, ngroups, d, f, intra;
};

__global__ __launch_bounds__(NTHREADS, 1) void k_out(OutArgs p) {
  __shared__ __attribute__((aligned(16))) Stage ring[NS];
  const int i0 = blockIdx.x * BM;
  const int j0 = blockIdx.y * BN;
  const int b = blockIdx.z / p.ngroups, g = blockIdx.z % p.ngroups;
  const long long gs = (long long)g * p.L;
  const int Lg = (int)((p.T - gs) < p.L ? (p.T - gs) : p.L);
  if (j0 >= Lg) return;
  const Opnd sa1 = rowmajor(p.snap + ((long long)b * p.ngroups + g) * p.d * p.f, p.f, p.d, p.f);
  const Opnd sb1 = rowmajor(p.Z + ((long long)b * p.T_pad + gs) * p.f, p.f, (int)(p.T_pad - gs), p.f);
  int nk2 = 0;
  Opnd sa2 = sa1, sb2 = sb1;
  if (p.intra) {
    const int jl = (j0 + BN - 1 < Lg - 1) ? j0 + BN - 1 : Lg - 1;
    const int kend = (jl / p.C) * p.C;  // start of the last row's chunk
    const int kv = (kend + 7) & ~7;
    nk2 = (kv + BK - 1) / BK;
    sa2 = kblocked(p.VT + (long long)b * p.d * p.T_pad, (long long)p.d * 64, p.d, kv, (int)gs);
    sb2 = rowmajor(p.P + ((long long)b * p.ngroups + g) * p.L * p.L, p.L, p.L, kv);
  }
  Acc acc;
  acc_zero(acc);
  gemm_loop<true>(acc, ring, sa1, sb1, p.f / BK, sa2, sb2, nk2, i0, j0);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) {
    const int t = j0 + wn * 128 + bj * 32 + (lane & 31);
    if (t >= Lg) continue;
    bf16_t *yrow = p.y + ((long long)b * p.T + gs + t) * p.d;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int a = i0 + wm * 128 + bi * 32 + 8 * q + 4 * (lane >> 5);
        uint2 pk;
        pk.x = pack_bf16x2(acc.v[bi][bj][4 * q + 0], acc.v[bi][bj][4 * q + 1]);
        pk.y = pack_bf16x2(acc.v[bi][bj][4 * q + 2], acc.v[bi][bj][4 * q + 3]);
        *reinterpret_cast<uint2 *>(yrow + a) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// Target gather, transposed and K-blocked: V^T[b][p/64][a][p%64] = E[ids[b][p+1]][a].
// A 64-slot x 64-feature tile passes through LDS so both the row reads of E and
// the writes (one contiguous 8 KB block) are 16 B per lane.
// grid: (T_pad/64, d/64, B)
__global__ __launch_bounds__(256) void k_gather_vt(const int32_t *ids, const bf16_t *E, int vocab, bf16_t *VT, int T,
                                                   int T_pad, int d) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64][72];
  const int p0 = blockIdx.x * 64, a0 = blockIdx.y * 64, b = blockIdx.z;
  const int tid = threadIdx.x, seg = tid & 7;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int pl = pass * 32 + (tid >> 3);
    const int pos = p0 + pl;
    int id = -1;
    if (pos < T) id = ids[(long long)b * (T + 1) + pos + 1];
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (id >= 0 && id < vocab) v = *reinterpret_cast<const uint4 *>(E + (long long)id * d + a0 + seg * 8);
    *reinterpret_cast<uint4 *>(&tile[pl][seg * 8]) = v;
  }
  __syncthreads();
  bf16_t *blk = VT + ((long long)b * (T_pad / 64) + blockIdx.x) * d * 64;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int al = pass * 32 + (tid >> 3);
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wv[e] = (uint32_t)tile[seg * 8 + 2 * e][al] | ((uint32_t)tile[seg * 8 + 2 * e + 1][al] << 16);
    *reinterpret_cast<uint4 *>(blk + (long long)(a0 + al) * 64 + seg * 8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

}  // namespace

hipError_t launch_gather_vt_bf16(const int32_t *ids, const bf16_t *E, int vocab, bf16_t *VT, const Layout &lay,
                                 hipStream_t s) {
  dim3 grid(lay.T_pad / 64, lay.d / 64, lay.B);
  hipLaunchKernelGGL(k_gather_vt, grid, dim3(256), 0, s, ids, E, vocab, VT, lay.T, lay.T_pad, lay.d);
  return hipGetLastError();
}

hipError_t launch_a1_bf16(const bf16_t *x, const bf16_t *Wug, bf16_t *Z, bf16_t *ZT, float eta, int write_zt,
                          const Layout &lay, hipStream_t s) {
  A1Args p{x, Wug, Z, ZT, eta, write_zt, lay.T, lay.T_pad, lay.d, lay.f};
  dim3 grid((2 * lay.f + BN - 1) / BN, (unsigned)((long long)lay.B * lay.T_pad / BM));
  hipLaunchKernelGGL(k_a1, grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_update_bf16(const bf16_t *ZT, const bf16_t *VT, float *state, bf16_t *snap, const Layout &lay,
                              hipStream_t s) {
  const int kend = (int)round_up_ll(lay.T, BK);
  UpdArgs p{ZT, VT, state, snap, lay.T_pad, kend, lay.L, lay.ngroups, lay.d, lay.f};
  dim3 grid(lay.f / BM, lay.d / BN, lay.B);
  hipLaunchKernelGGL(k_update, grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_scores_bf16(const bf16_t *Z, bf16_t *P, float eta, const Layout &lay, hipStream_t s) {
  const int nt = (lay.L + BN - 1) / BN;
  ScoreArgs p{Z, P, eta, lay.T, lay.T_pad, lay.L, lay.C, lay.ngroups, lay.f, nt};
  dim3 grid(nt * nt, lay.ngroups, lay.B);
  hipLaunchKernelGGL(k_scores, grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_out_bf16(const bf16_t *Z, const bf16_t *P, const bf16_t *snap, const bf16_t *VT, bf16_t *y,
                           const Layout &lay, hipStream_t s) {
  OutArgs p{Z, P, snap, VT, y, lay.T, lay.T_pad, lay.L, lay.C, lay.ngroups, lay.d, lay.f, lay.intra};
  dim3 grid(lay.d / BM, (lay.L + BN - 1) / BN, lay.B * lay.ngroups);
  hipLaunchKernelGGL(k_out, grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}
