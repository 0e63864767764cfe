// bf16 MFMA kernels of the chunk-wise fast-weight path (gfx950).
//
// Every contraction is written as D[i][j] = sum_k A[i][k] * B[j][k] with both
// operands K-contiguous in HBM ("NT" form). A block computes a 256 x 256 tile
// with 4 waves (2 x 2), each wave 128 x 128 as 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators. K advances in steps of 64
// through two LDS stages (64 KB each). Tiles go from HBM straight into LDS with
// 16-byte buffer loads (no register staging); 16-byte chunks of each LDS row
// are XOR-swizzled so that the MFMA fragment reads are free of bank conflicts.
// Rows or columns outside an operand's valid range are loaded through an
// out-of-range buffer offset, which the hardware returns as zero.
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
constexpr int BK = 64;   // k per stage
constexpr int NTHREADS = 256;
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer descriptor word 3 on the gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;   // offset past num_records: the load returns zero

struct Acc {
  f32x16 v[4][4];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// element offset of (row r, 16-byte chunk c) inside a ROWS x 64 bf16 LDS tile
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }

__device__ __forceinline__ void acc_zero(Acc &acc) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.v[bi][bj][r] = 0.f;
}

// Queue the copy of rows [row0, row0+256) x cols [k, k+64) of one segment into
// an LDS tile. Wave w moves rows w*64 .. w*64+63, eight rows per instruction;
// lane l of an instruction fills row r0 + l/8, physical chunk l%8, so it loads
// the logical chunk (l%8) ^ swz(row). One descriptor covers the tile; the
// slab's row offset goes in soffset. Row pitches stay below 2^24 bytes, so all
// offsets fit in 31 bits.
__device__ __forceinline__ void issue_tile(bf16_t *lds_tile, const Seg<bf16_t> &s, int row0, int k, int w,
                                           int lane) {
  const int lr = lane >> 3;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(s.base + (long long)row0 * s.ld + k), (short)0, 0x7fffffff, kBufferFlags);
  const int ldb = (int)s.ld * 2;           // row pitch in bytes
  const int nvw = s.nrows - row0 - w * 64;  // valid rows among this wave's 64
  const int kleft = s.kvalid - k;          // valid columns from k on
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int c = (lane & 7) ^ lr ^ (n & 1);
    const bool ok = (n * 8 + lr) < nvw && c * 8 < kleft;
    const uint32_t voff = ok ? (uint32_t)(lr * ldb + c * 16) : kOutOfRange;
    const int slab = w * 64 + n * 8;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lds_tile + slab * BK), 16, voff, slab * ldb, 0, 0);
  }
}

// Wait for this wave's queued tile loads, then for every wave.
__device__ __forceinline__ void stage_ready() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// One 64-deep stage: 4 k-substeps of 16, 16 MFMAs each. When MASKED, only the
// 8-element k groups g with glo <= g < ghi (g = 0..7 within the stage) count.
template <bool MASKED>
__device__ __forceinline__ void mma_stage(Acc &acc, const bf16_t *lA, const bf16_t *lB, int wm, int wn, int lane,
                                          int glo = 0, int ghi = 8) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = 2 * ks + (lane >> 5);
    bf16x8 a[4], b[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
      a[bi] = *reinterpret_cast<const bf16x8 *>(lA + lds_off(wm * 128 + bi * 32 + (lane & 31), c));
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
      b[bj] = *reinterpret_cast<const bf16x8 *>(lB + lds_off(wn * 128 + bj * 32 + (lane & 31), c));
    if (MASKED) {
      if (c < glo || c >= ghi) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) b[bj] = bf16x8{};
      }
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
        acc.v[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc.v[bi][bj], 0, 0, 0);
  }
}

typedef bf16_t LdsStage[2][BM * BK];  // [operand A/B][tile]

// K loop over segment 1 (nk1 stages) then segment 2 (nk2 stages).
__device__ __forceinline__ void gemm_loop(Acc &acc, LdsStage *lds, const Seg<bf16_t> &sa1, const Seg<bf16_t> &sb1,
                                          int nk1, const Seg<bf16_t> &sa2, const Seg<bf16_t> &sb2, int nk2,
                                          int arow0, int brow0) {
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1, wn = w & 1;
  const int nk = nk1 + nk2;
  if (nk <= 0) return;
  auto issue = [&](int kt, int buf) {
    if (kt < nk1) {
      issue_tile(lds[buf][0], sa1, arow0, kt * BK, w, lane);
      issue_tile(lds[buf][1], sb1, brow0, kt * BK, w, lane);
    } else {
      issue_tile(lds[buf][0], sa2, arow0, (kt - nk1) * BK, w, lane);
      issue_tile(lds[buf][1], sb2, brow0, (kt - nk1) * BK, w, lane);
    }
  };
  issue(0, 0);
  stage_ready();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
    mma_stage<false>(acc, lds[cur][0], lds[cur][1], wm, wn, lane);
    stage_ready();
  }
}

// ---------------------------------------------------------------------------
// Up/gate GEMM with SwiGLU epilogue. i = token slot, j = interleaved W_ug row.
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
  __shared__ __attribute__((aligned(16))) LdsStage lds[2];
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int b = m0 / p.T_pad;
  const int pos0 = m0 - b * p.T_pad;
  const int valid_rows = p.T - pos0;  // x rows >= T read as zero
  Seg<bf16_t> sa{p.x + ((long long)b * p.T + pos0) * p.d, p.d, valid_rows, p.d};
  Seg<bf16_t> sb{p.Wug + (long long)n0 * p.d, p.d, 2 * p.f - n0, p.d};
  Acc acc;
  acc_zero(acc);
  gemm_loop(acc, lds, sa, sb, p.d / BK, sa, sb, 0, 0, 0);

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1, wn = w & 1;
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
          *reinterpret_cast<uint2 *>(p.ZT + ((long long)b * p.f + feat) * p.T_pad + pos) = pk;
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
  __shared__ __attribute__((aligned(16))) LdsStage lds[2];
  const int i0 = blockIdx.x * BM;
  const int j0 = blockIdx.y * BN;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1, wn = w & 1;
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
    __builtin_amdgcn_sched_barrier(0);  // one column block at a time: bounded register use
  }

  Seg<bf16_t> sa{p.ZT + (long long)b * p.f * p.T_pad, p.T_pad, p.f, p.T_pad};
  Seg<bf16_t> sb{p.VT + (long long)b * p.d * p.T_pad, p.T_pad, p.d, p.T_pad};
  const int nk = p.kend / BK;
  if (nk > 0) {
    issue_tile(lds[0][0], sa, i0, 0, w, lane);
    issue_tile(lds[0][1], sb, j0, 0, w, lane);
    stage_ready();
  }
  // One pass per (stage, part): a group start g*L inside stage [k0, k0+64)
  // ends the current part there; the tile is written out as snapshot g and
  // the same stage continues from that k group.
  int kt = 0, glo = 0, g = 0;
  bool issued = false;
  while (kt < nk) {
    const int cur = kt & 1;
    const int k0 = kt * BK;
    if (!issued) {
      if (kt + 1 < nk) {
        issue_tile(lds[cur ^ 1][0], sa, i0, k0 + BK, w, lane);
        issue_tile(lds[cur ^ 1][1], sb, j0, k0 + BK, w, lane);
      }
      issued = true;
    }
    const bool boundary = g < p.ngroups && (long long)g * p.L < k0 + BK;
    const int ghi = boundary ? (int)((long long)g * p.L - k0) >> 3 : 8;
    if (ghi > glo) mma_stage<true>(acc, lds[cur][0], lds[cur][1], wm, wn, lane, glo, ghi);
    if (boundary) {
      dump_snapshot(acc, snap0 + (long long)g * df, p.f);
      ++g;
      glo = ghi;
    } else {
      stage_ready();
      ++kt;
      glo = 0;
      issued = false;
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
  __shared__ __attribute__((aligned(16))) LdsStage lds[2];
  const int it = blockIdx.x % p.nt, jt = blockIdx.x / p.nt;
  const int g = blockIdx.y, b = blockIdx.z;
  const long long gs = (long long)g * p.L;
  const int Lg = (int)((p.T - gs) < p.L ? (p.T - gs) : p.L);
  const int i0 = it * BM, j0 = jt * BN;
  if (it > jt || j0 >= Lg) return;
  const bf16_t *Zg = p.Z + ((long long)b * p.T_pad + gs) * p.f;
  const int rows = (int)(p.T_pad - gs);
  Seg<bf16_t> sa{Zg, p.f, rows, p.f};
  Seg<bf16_t> sb{Zg, p.f, rows, p.f};
  Acc acc;
  acc_zero(acc);
  gemm_loop(acc, lds, sa, sb, p.f / BK, sa, sb, 0, i0, j0);

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1, wn = w & 1;
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
        const int s = i0 + wm * 128 + bi * 32 + 8 * q + 4 * (lane >> 5);
        if (s >= p.L) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = ((s + r) / p.C < ct) ? p.eta * acc.v[bi][bj][4 * q + r] : 0.f;
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(Pg + (long long)t * p.L + s) = pk;
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
  __shared__ __attribute__((aligned(16))) LdsStage lds[2];
  const int i0 = blockIdx.x * BM;
  const int j0 = blockIdx.y * BN;
  const int b = blockIdx.z / p.ngroups, g = blockIdx.z % p.ngroups;
  const long long gs = (long long)g * p.L;
  const int Lg = (int)((p.T - gs) < p.L ? (p.T - gs) : p.L);
  if (j0 >= Lg) return;
  Seg<bf16_t> sa1{p.snap + ((long long)b * p.ngroups + g) * p.d * p.f, p.f, p.d, p.f};
  Seg<bf16_t> sb1{p.Z + ((long long)b * p.T_pad + gs) * p.f, p.f, (int)(p.T_pad - gs), p.f};
  int nk2 = 0;
  Seg<bf16_t> sa2 = sa1, sb2 = sb1;
  if (p.intra) {
    const int jl = (j0 + BN - 1 < Lg - 1) ? j0 + BN - 1 : Lg - 1;
    const int kend = (jl / p.C) * p.C;  // start of the last row's chunk
    const int kv = (kend + 7) & ~7;
    nk2 = (kv + BK - 1) / BK;
    sa2 = Seg<bf16_t>{p.VT + (long long)b * p.d * p.T_pad + gs, p.T_pad, p.d, kv};
    sb2 = Seg<bf16_t>{p.P + ((long long)b * p.ngroups + g) * p.L * p.L, p.L, p.L, kv};
  }
  Acc acc;
  acc_zero(acc);
  gemm_loop(acc, lds, sa1, sb1, p.f / BK, sa2, sb2, nk2, i0, j0);

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1, wn = w & 1;
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
        if (a >= p.d) continue;
        uint2 pk;
        pk.x = pack_bf16x2(acc.v[bi][bj][4 * q + 0], acc.v[bi][bj][4 * q + 1]);
        pk.y = pack_bf16x2(acc.v[bi][bj][4 * q + 2], acc.v[bi][bj][4 * q + 3]);
        *reinterpret_cast<uint2 *>(yrow + a) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// Target gather, transposed: V^T[b][a][p]. A 64-slot x 64-feature tile passes
// through LDS so both the row reads of E and the row writes of V^T are 16 B.
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
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int al = pass * 32 + (tid >> 3);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[seg * 8 + 2 * e][al] | ((uint32_t)tile[seg * 8 + 2 * e + 1][al] << 16);
    *reinterpret_cast<uint4 *>(VT + ((long long)b * d + a0 + al) * T_pad + p0 + seg * 8) =
        make_uint4(w[0], w[1], w[2], w[3]);
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
  dim3 grid((lay.f + BM - 1) / BM, (lay.d + BN - 1) / BN, lay.B);
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
  dim3 grid((lay.d + BM - 1) / BM, (lay.L + BN - 1) / BN, lay.B * lay.ngroups);
  hipLaunchKernelGGL(k_out, grid, dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}
