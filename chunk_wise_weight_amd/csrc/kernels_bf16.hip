// bf16 MFMA kernels of the chunk-wise fast-weight path (gfx950).
//
// Every contraction is written as D[i][j] = sum_k A[i][k] * B[j][k] with both
// operands K-contiguous ("NT" form). A block has 2 x WN waves; each wave
// computes 128 x (32*NBJ) with v_mfma_f32_32x32x16_bf16 and fp32 accumulators
// in AGPRs. Every GEMM uses 8 waves (WN = 4, NBJ = 2: 256 x 256 tiles, two
// waves per SIMD so one can issue MFMAs while the other waits), except the
// last, partial round of the state update, which runs 256 x 128 halves on 4
// waves (WN = 2, NBJ = 2).
//
// Tiles go from HBM straight into LDS with 16-byte buffer loads (no register
// staging) in slabs of 64 columns, so that every row contributes one whole
// 128-byte line: whole lines fill LDS at twice the rate of half lines. A ring
// of NSL slabs keeps the next slabs in flight while one is multiplied, and
// each wave waits only for the oldest slab it needs. The MFMAs run in stages
// of 32 (two per slab); within a stage the fragment reads of the next
// k-substep and the next stage are issued behind MFMAs already queued (a
// software pipeline). The eight 16-byte chunks of each 128-byte LDS row are
// XOR-swizzled so that the fragment reads are free of bank conflicts. Rows or
// columns outside an operand's valid range are fetched through an
// out-of-range buffer offset, which the hardware returns as zero.
//
// Operands are row-major (element (r, k) at r*ld + k), K-blocked by 64
// (element (r, k) at (k/64)*kblk + r*64 + k%64), or held in planes of 8
// columns (element (r, k) at (k/8)*pstride + r*8 + k%8). V^T and Z are
// K-blocked (Z's blocks hold every token slot, [f/64][T_pad][64]), so one slab
// of a tile is one contiguous block instead of rows strided by the whole
// stream length or by f. eta*Z^T and the snapshots are planes: the MFMA register layout holds
// four consecutive k of one row per lane, so a store instruction of 32 rows x
// 16 bytes is 512 contiguous bytes in a plane (in row-major or K-blocked form
// it would touch 32 lines); a plane slab loads as 1 KB contiguous pieces into
// an LDS tile of [8][256][8], whose fragment reads need no swizzle.
//
// MFMA 32x32x16 register layout (lane l, accumulator register r):
//   A operand: row i = l % 32, k = 8*(l/32) .. +7;  B operand: column j = l % 32, same k.
//   D: j = l % 32, i = 8*(r/4) + 4*(l/32) + r%4.
// So each lane holds, per group of 4 registers, four consecutive i for one j:
// epilogues store 4 consecutive elements along i.
#include <type_traits>

#include "launch.h"

namespace {

constexpr int BM = 256;  // tile rows along i
constexpr int BK = 32;   // k per MFMA stage
constexpr int SK = 64;   // k per load slab: one 128-byte line of every row
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer descriptor word 3 on the gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;   // offset past num_records: the load returns zero

template <int NBJ>
struct Acc {
  f32x16 v[4][NBJ];
};

// One LDS slab: the A tile (256 rows) and the B tile (32*WN*NBJ rows), 64 columns each.
template <int WN, int NBJ>
struct Slab {
  bf16_t a[BM * SK];
  bf16_t b[32 * WN * NBJ * SK];
};

typedef __attribute__((address_space(3))) void lds_void;

// The eight 16-byte chunks of each 128-byte LDS row are XOR-swizzled; with
// this pattern the fragment reads (32 consecutive rows, one chunk) are free of
// bank conflicts, also while LDS-DMA writes land (measured with rocprofv3).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
// element offset of (row r, logical 16-byte chunk c) inside an N x 64 bf16 LDS tile
__device__ __forceinline__ int lds_off(int r, int c) { return r * SK + ((c ^ swz(r)) << 3); }

template <int NBJ>
__device__ __forceinline__ void acc_zero(Acc<NBJ> &acc) {
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.v[bi][bj][r] = 0.f;
}

// buffer loads per wave per slab: A tile, then B tile
template <int WN, int NBJ>
constexpr int loads_a() { return BM / (2 * WN) / 8; }
template <int WN, int NBJ>
constexpr int loads_per_slab() { return loads_a<WN, NBJ>() + 32 * WN * NBJ / (2 * WN) / 8; }

// ---- Tile loads ----
// A load instruction moves 1 KB from memory straight into LDS: 16 bytes per
// lane, lane l landing at the instruction's LDS base + 16 l. Descriptors and
// per-lane offsets are prepared once (per tile, or per slab where the slab
// moves the base), so each load costs one instruction and a scalar offset.
//
// Row-major and K-blocked tiles load 8 rows per instruction: lanes 8r .. 8r+7
// fetch the whole 128-byte line of row r (whole lines fill LDS at twice the
// rate of half lines), and lane l fills physical chunk l%8, i.e. the logical
// chunk (l%8) ^ swz(row). Load n of wave w (of NW) moves rows
// w*ROWS/NW + 8n .. +8.

// Row-major operand: element (r, k) at base[r*ld + k], base at the tile's
// first row. Rows r >= nrows read zero: the lane offset holds the whole row
// offset and passes num_records. COLS: columns >= kvalid read zero too.
template <int ROWS, int NW, bool COLS = false>
struct RmLoad {
  static constexpr int WR = ROWS / NW, N = WR / 8;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo[N];
  int kvalid;
  __device__ __forceinline__ void init(const bf16_t *base, long long ld, int nrows, int kvalid_, int w, int lane) {
    const long long bytes = (long long)(nrows > 0 ? nrows : 0) * ld * 2;
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(base), (short)0,
                                           (int)(bytes < 0x7fffffffLL ? bytes : 0x7fffffffLL), kBufferFlags);
    kvalid = kvalid_;
    const int lr = lane >> 3;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int row = w * WR + 8 * n + lr;
      vo[n] = (uint32_t)((long long)row * ld * 2 + (((lane & 7) ^ swz(row)) << 4));
    }
  }
  struct Pre {};
  __device__ __forceinline__ Pre prep(int) const { return Pre{}; }
  __device__ __forceinline__ void issue(const Pre &, bf16_t *tile, int sl, int w, int lane, int n) const {
    uint32_t v = vo[n];
    if (COLS) {
      const int c = (lane & 7) ^ swz(w * WR + 8 * n + (lane >> 3));
      if (sl * SK + c * 8 >= kvalid) v = kOutOfRange;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (w * WR + 8 * n) * SK), 16, v, sl * SK * 2, 0,
                                             0);
  }
};

// Column-blocked operand [K/64][rows][64]: element (r, k) at
// base[(k/64)*kblk + r*64 + k%64], base at the tile's first row in block 0.
// Each slab is one contiguous block of 128-byte rows; its descriptor starts at
// the slab's block and ends after nrows rows, so rows r >= nrows read zero
// (the row offset is in the lane offset, which the range check covers).
template <int ROWS, int NW>
struct CbLoad {
  static constexpr int WR = ROWS / NW, N = WR / 8;
  const bf16_t *base;
  long long kblk;
  int bytes;
  // a fixed bound: with vo[N] here, the host pass of hipcc rejects SlabLoads<PlLoad, CbLoad>
  uint32_t vo[8];
  static_assert(N <= 8, "lane offsets per wave");
  __device__ __forceinline__ void init(const bf16_t *base_, long long kblk_, int nrows, int w, int lane) {
    base = base_;
    kblk = kblk_;
    const long long by = (long long)(nrows > 0 ? nrows : 0) * 128;
    bytes = (int)(by < 0x7fffffffLL ? by : 0x7fffffffLL);
    const int lr = lane >> 3;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int row = w * WR + 8 * n + lr;
      vo[n] = (uint32_t)(row * 128 + (((lane & 7) ^ swz(row)) << 4));
    }
  }
  using Pre = __amdgpu_buffer_rsrc_t;
  __device__ __forceinline__ Pre prep(int sl) const {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(base + (long long)sl * kblk), (short)0, bytes,
                                             kBufferFlags);
  }
  __device__ __forceinline__ void issue(const Pre &rs, bf16_t *tile, int, int w, int, int n) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (w * WR + 8 * n) * SK), 16, vo[n], 0, 0, 0);
  }
};

// Gathered rows: row r of the operand is row rid[r] of a row-major table E
// ([nrows_e][ld], nrows_e*ld*2 < 2^31 bytes); rows r >= nvalid, and rows whose
// id falls outside [0, nrows_e), read zero.
template <int ROWS, int NW>
struct RmGather {
  static constexpr int WR = ROWS / NW, N = WR / 8;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo[N];
  __device__ __forceinline__ void init(const bf16_t *E, int ld, int nrows_e, const int32_t *rid, int nvalid, int w,
                                       int lane) {
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(E), (short)0, (int)((long long)nrows_e * ld * 2),
                                           kBufferFlags);
    const int lr = lane >> 3;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int row = w * WR + 8 * n + lr;
      const int id = row < nvalid ? rid[row] : -1;
      vo[n] = (id >= 0 && id < nrows_e) ? (uint32_t)id * (uint32_t)ld * 2u + (uint32_t)(((lane & 7) ^ swz(row)) << 4)
                                        : kOutOfRange;
    }
  }
  struct Pre {};
  __device__ __forceinline__ Pre prep(int) const { return Pre{}; }
  __device__ __forceinline__ void issue(const Pre &, bf16_t *tile, int sl, int w, int, int n) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (w * WR + 8 * n) * SK), 16, vo[n], sl * SK * 2, 0,
                                             0);
  }
};

// K-blocked operand: element (r, k) at base[(k/64)*kblk + r*64 + k%64], base
// at the tile's first row in block 0; every row of the tile is valid. The
// descriptor follows the slab's block. The swizzle depends on n only through
// its parity (WR is a multiple of 16), so two lane offsets serve every load.
template <int ROWS, int NW>
struct KbLoad {
  static constexpr int WR = ROWS / NW, N = WR / 8;
  static_assert(WR % 16 == 0, "two lane offsets need WR a multiple of 16");
  const bf16_t *base;
  long long kblk;
  uint32_t ve, vd;  // lane offsets for even / odd n
  __device__ __forceinline__ void init(const bf16_t *base_, long long kblk_, int w, int lane) {
    base = base_;
    kblk = kblk_;
    const int lr = lane >> 3;
    ve = (uint32_t)(lr * 128 + (((lane & 7) ^ swz(w * WR + lr)) << 4));
    vd = (uint32_t)(lr * 128 + (((lane & 7) ^ swz(w * WR + 8 + lr)) << 4));
  }
  using Pre = __amdgpu_buffer_rsrc_t;
  __device__ __forceinline__ Pre prep(int sl) const {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(base + (long long)sl * kblk), (short)0, 0x7fffffff,
                                             kBufferFlags);
  }
  __device__ __forceinline__ void issue(const Pre &rs, bf16_t *tile, int, int w, int, int n) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (w * WR + 8 * n) * SK), 16, (n & 1) ? vd : ve,
                                             (w * WR + 8 * n) * 128, 0, 0);
  }
};

// Plane operand (planes of 8 columns): element (r, k) at base[(k/8)*pstride +
// r*8 + k%8], base at the tile's first row in plane 0; 256-row tiles, every
// row valid. Load n of wave w moves 1 KB piece q = w*(32/NW) + n of the slab:
// rows (q%4)*64 .. +64 of plane q/4, contiguous in memory and in the LDS tile
// [8 planes][256 rows][8].
template <int NW>
struct PlLoad {
  static constexpr int N = 32 / NW;
  const bf16_t *base;
  long long pstride;
  uint32_t vl;  // lane * 16
  __device__ __forceinline__ void init(const bf16_t *base_, long long pstride_, int lane) {
    base = base_;
    pstride = pstride_;
    vl = (uint32_t)(lane * 16);
  }
  using Pre = __amdgpu_buffer_rsrc_t;
  __device__ __forceinline__ Pre prep(int sl) const {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(base + (long long)sl * 8 * pstride), (short)0,
                                             0x7fffffff, kBufferFlags);
  }
  // N is a multiple of 4, so the row block is q%4 = n%4
  __device__ __forceinline__ void issue(const Pre &rs, bf16_t *tile, int, int w, int, int n) const {
    static_assert(N % 4 == 0, "row block from n alone");
    const int pl = w * (N / 4) + (n >> 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(tile + (pl * BM + (n & 3) * 64) * 8), 16, vl,
                                             (int)(pl * pstride * 2) + (n & 3) * 1024, 0, 0);
  }
};

// The loads of one slab: the A tile's, then the B tile's.
template <class LA, class LB>
struct SlabLoads {
  LA a;
  LB b;
  static constexpr int N = LA::N + LB::N;
  static constexpr bool kPf = false;  // no prefetch
  struct Pre {
    typename LA::Pre a;
    typename LB::Pre b;
  };
  __device__ __forceinline__ Pre prep(int sl) const { return Pre{a.prep(sl), b.prep(sl)}; }
  template <class S>
  __device__ __forceinline__ void issue(const Pre &p, S &slab, int sl, int w, int lane, int j) const {
    if (j < LA::N)
      a.issue(p.a, slab.a, sl, w, lane, j);
    else
      b.issue(p.b, slab.b, sl, w, lane, j - LA::N);
  }
};

// s_waitcnt immediate (gfx9): vmcnt(n), expcnt unchanged, lgkmcnt(0).
constexpr unsigned wait_imm(int n) { return (unsigned)((n & 15) | 0x70 | (((n >> 4) & 3) << 14)); }

// Wait until at most `later` slabs of this wave's loads (LPS loads per slab)
// are still in flight and its own LDS reads are done, then meet every wave at
// the barrier: their loads of the awaited slab have landed too, and every
// wave is done reading the slab computed before. Only LDS is shared between
// the waves, so no memory fence is needed (a fence would also wait for the
// loads of the slabs still in flight). `later` is at most MAXL. EXTRA more
// operations issued after the awaited slab's loads (prefetches) may stay in
// flight too: the counter is decremented in issue order.
template <int LPS, int MAXL, int EXTRA = 0>
__device__ __forceinline__ void slab_wait(int later) {
  static_assert(MAXL >= 0 && MAXL <= 2 && MAXL * LPS + EXTRA <= 63, "vmcnt holds 6 bits");
  if (MAXL == 0 || later <= 0)
    __builtin_amdgcn_s_waitcnt(wait_imm(EXTRA));
  else if (MAXL == 1 || later == 1)
    __builtin_amdgcn_s_waitcnt(wait_imm((MAXL >= 1 ? LPS : 0) + EXTRA));
  else
    __builtin_amdgcn_s_waitcnt(wait_imm(MAXL * LPS + EXTRA));
  asm volatile("s_barrier" ::: "memory");
}

// MFMA fragments of one 16-deep k-substep: 4 A fragments (rows) and NBJ B
// fragments (columns) of this wave's sub-tile.
template <int NBJ>
struct Frag {
  bf16x8 a[4], b[NBJ];
};

// Read substep ks (0 or 1) of half h (0 or 1) of an LDS slab into registers.
// APLANE: the A tile is held as 8 planes of [256 rows][8 columns] (column
// chunk c of row r at (c*256 + r)*8) instead of swizzled 128-byte rows.
template <int WN, int NBJ, bool APLANE = false>
__device__ __forceinline__ void frag_read(Frag<NBJ> &fr, const Slab<WN, NBJ> &st, int h, int ks, int wm, int wn,
                                          int lane) {
  const int c = 4 * h + 2 * ks + (lane >> 5);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
    fr.a[bi] = *reinterpret_cast<const bf16x8 *>(
        st.a + (APLANE ? (c * BM + wm * 128 + bi * 32 + (lane & 31)) * 8 : lds_off(wm * 128 + bi * 32 + (lane & 31), c)));
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj)
    fr.b[bj] = *reinterpret_cast<const bf16x8 *>(st.b + lds_off(wn * 32 * NBJ + bj * 32 + (lane & 31), c));
}

// MFMAs of one k-substep for fragment rows bi in [BLO, BHI).
template <int BLO, int BHI, int NBJ>
__device__ __forceinline__ void frag_mma(Acc<NBJ> &acc, const Frag<NBJ> &fr) {
#pragma unroll
  for (int bi = BLO; bi < BHI; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj)
      acc.v[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[bi], fr.b[bj], acc.v[bi][bj], 0, 0, 0);
}

// Keep the compiler from moving instructions across this point.
__device__ __forceinline__ void pin() { __builtin_amdgcn_sched_barrier(0); }

// Issue point P (0..6) of a stage that refills a slab: loads [P*LPS/7, (P+1)*LPS/7).
template <int LPS, int P, class SL, class S>
__device__ __forceinline__ void issue_point(const SL &ld, const typename SL::Pre &pre, S &slab, int sl, int w,
                                            int lane) {
#pragma unroll
  for (int j = P * LPS / 7; j < (P + 1) * LPS / 7; ++j) ld.issue(pre, slab, sl, w, lane, j);
}

// The software pipeline of one 32-deep stage kt = half kt%2 of slab kt/2. On
// entry `cur` holds (or is loading) substep 0 of stage kt; on exit it holds
// substep 0 of stage kt+1. Every LDS read and tile-load issue sits behind
// MFMAs already queued, so the matrix cores keep running while they wait:
//   read substep 1 of kt -> nxt | MFMAs of row 0 on cur
//   at the end of a slab: wait for the next slab + barrier
//   MFMAs of rows 1-3 on cur and rows 0-3 on nxt, with this wave's loads of
//   slab kt/2 + NSL (into the buffer just finished) issued between them, and
//   substep 0 of kt+1 read into cur after nxt's first row.
// After the barrier no wave reads the finished slab's buffer again (all its
// reads were issued before, and the wait includes lgkmcnt(0)), so it can be
// refilled. Spreading the loads keeps a burst of them from stalling the MFMA
// issue. With AFTER, after_fn(acc) runs once all of stage kt's MFMAs are
// queued, and the next fragments are read only then (few registers live).
// Loads with a prefetch (SL::kPf) also touch, in every odd stage, this
// workgroup's share of slab kt/2 + NSL + 2, so that the slab's own loads two
// stages later find it in L2.
// H (= kt % 2) and REFILL (this stage refills the buffer it finished: 1/0)
// are fixed at compile time where the caller knows them, else -1 (decided
// here at run time).
template <int WN, int NBJ, int NSL, bool AFTER, bool APLANE, int H, int REFILL, class SL, class AfterFn>
__device__ __forceinline__ void stage_body(Acc<NBJ> &acc, Slab<WN, NBJ> *ring, Frag<NBJ> &cur, Frag<NBJ> &nxt,
                                           int kt, int nk, int wm, int wn, int lane, int w, const SL &ld,
                                           AfterFn &&after_fn) {
  constexpr int LPS = loads_per_slab<WN, NBJ>();
  static_assert(SL::N == LPS, "the slab loads match the tile configuration");
  const int sl = kt >> 1;
  const int nsl = (nk + 1) >> 1;
  const int h = H >= 0 ? H : (kt & 1);
  const bool refill = REFILL >= 0 ? REFILL == 1 : (h == 1 && sl + NSL < nsl);
  frag_read<WN, NBJ, APLANE>(nxt, ring[sl % NSL], h, 1, wm, wn, lane);
  pin();
  frag_mma<0, 1>(acc, cur);
  pin();
  const bool more = kt + 1 < nk;  // always true when refilling
  if (h == 1 && (refill || more)) {
    const int later = (nsl - 2 - sl) < (NSL - 2) ? (nsl - 2 - sl) : (NSL - 2);
    slab_wait<LPS, NSL - 2, SL::kPf ? 1 : 0>(later);
  }
  const int rs = sl + NSL;
  Slab<WN, NBJ> &dst = ring[sl % NSL];  // the buffer just finished refills with slab rs
  typename SL::Pre pre{};
  if (refill) pre = ld.prep(rs);
  pin();
  frag_mma<1, 2>(acc, cur);
  if (refill) issue_point<LPS, 0>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<2, 3>(acc, cur);
  if (refill) issue_point<LPS, 1>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<3, 4>(acc, cur);
  if (refill) issue_point<LPS, 2>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<0, 1>(acc, nxt);
  pin();
  // unconditional (past the end it reads a stale buffer of the ring): no
  // branch, so the compiler can count the reads and wait for each exactly
  if (!AFTER) frag_read<WN, NBJ, APLANE>(cur, ring[((kt + 1) >> 1) % NSL], (kt + 1) & 1, 0, wm, wn, lane);
  if (refill) issue_point<LPS, 3>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<1, 2>(acc, nxt);
  if (refill) issue_point<LPS, 4>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<2, 3>(acc, nxt);
  if (refill) issue_point<LPS, 5>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<3, 4>(acc, nxt);
  if (refill) issue_point<LPS, 6>(ld, pre, dst, rs, w, lane);
  // one prefetch per odd stage, always issued, so every slab wait counts one
  if constexpr (SL::kPf) {
    if (h == 1) ld.prefetch((sl + NSL + 2) < (nsl - 1) ? (sl + NSL + 2) : (nsl - 1), w, lane);
  }
  pin();
  if (AFTER) {
    after_fn(acc);
    frag_read<WN, NBJ, APLANE>(cur, ring[((kt + 1) >> 1) % NSL], (kt + 1) & 1, 0, wm, wn, lane);
    pin();
  }
}

template <int WN, int NBJ, int NSL, bool AFTER, bool APLANE = false, class SL, class AfterFn>
__device__ __forceinline__ void pipelined_stage(Acc<NBJ> &acc, Slab<WN, NBJ> *ring, Frag<NBJ> &cur, Frag<NBJ> &nxt,
                                                int kt, int nk, int wm, int wn, int lane, int w, const SL &ld,
                                                AfterFn &&after_fn) {
  stage_body<WN, NBJ, NSL, AFTER, APLANE, -1, -1>(acc, ring, cur, nxt, kt, nk, wm, wn, lane, w, ld, after_fn);
}

struct NoHook {
  template <class A>
  __device__ void operator()(const A &) const {}
};

constexpr int WN_W = 4, NBJ_W = 2;  // wide GEMMs: 8 waves, 256 x 256 tiles
constexpr int NSL_W = 2;             // 2 x 64 KB slabs
constexpr int NT_W = 64 * 2 * WN_W;  // 512 threads
constexpr int WC_W = 32 * NBJ_W;     // columns per wave
constexpr int WN_U = 2, NBJ_U = 2;   // the state update's half-tile round: 4 waves, 256 x 128 tiles
constexpr int NSL_U = 3;             // 3 x 48 KB slabs
constexpr int NT_U = 64 * 2 * WN_U;  // 256 threads

// LDS of the output GEMM: the K-loop ring, reused by the epilogue to turn the
// MFMA register layout into whole-line stores of y.
constexpr int LY_P = 264;  // [256 tokens][256 model dims + pad]: y
constexpr int kRingBytes = (int)sizeof(Slab<WN_W, NBJ_W>) * NSL_W;
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kSmemOut = cmax(kRingBytes, 256 * LY_P * 2);

// wave coordinates: wm selects the 128-row half along i, wn the column slice along j
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Workgroups of a launch are handed to the 8 XCDs round-robin (workgroup n to
// XCD n % 8), and each XCD has its own L2. Renumber them so that XCD k works
// through one contiguous range of the logical tile order: the workgroups
// resident on an XCD at one time are then neighbours in that order and share
// operand tiles in its L2. A bijection on [0, N).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int n, int N) {
  const int xcd = n % kXcds, m = n / kXcds;
  const int q = N / kXcds, r = N % kXcds;
  return xcd * q + (xcd < r ? xcd : r) + m;
}

// Logical tile t of an nx x ny grid, in bands of H rows along y; inside a band
// y runs fastest, so H consecutive tiles share one x and nx*H consecutive tiles
// cover the band. The last band may be shorter.
__device__ __forceinline__ void band_tile(int t, int nx, int ny, int H, int &x, int &y) {
  const int full = ny / H, per = H * nx;
  const int band = t / per;
  const int h = band < full ? H : ny - full * H;
  const int r = t - band * per;
  x = r / h;
  y = band * H + r % h;
}

// Stages kt .. kt_end-1 of an nk-stage K loop without hooks (kt even), with
// each stage's parity and refill fixed at compile time: the stages of slabs
// 0 .. nsl-NSL-1 refill their buffer, the rest drain the ring, and an odd
// count of stages ends on a lone even stage. Leaves kt = kt_end.
template <int WN, int NBJ, int NSL, bool APLANE, class SL>
__device__ __forceinline__ void stage_run(Acc<NBJ> &acc, Slab<WN, NBJ> *ring, Frag<NBJ> &cur, Frag<NBJ> &nxt,
                                          int &kt, int kt_end, int nk, int wm, int wn, int lane, int w,
                                          const SL &ld) {
  const int nsl = (nk + 1) >> 1;
  const int kref = nsl > NSL ? 2 * (nsl - NSL) : 0;  // first stage past the refilling slabs
  const int k1 = kref < kt_end ? kref : kt_end;
  for (; kt + 1 < k1; kt += 2) {
    stage_body<WN, NBJ, NSL, false, APLANE, 0, 0>(acc, ring, cur, nxt, kt, nk, wm, wn, lane, w, ld, NoHook{});
    stage_body<WN, NBJ, NSL, false, APLANE, 1, 1>(acc, ring, cur, nxt, kt + 1, nk, wm, wn, lane, w, ld, NoHook{});
  }
  for (; kt + 1 < kt_end; kt += 2) {
    stage_body<WN, NBJ, NSL, false, APLANE, 0, 0>(acc, ring, cur, nxt, kt, nk, wm, wn, lane, w, ld, NoHook{});
    stage_body<WN, NBJ, NSL, false, APLANE, 1, 0>(acc, ring, cur, nxt, kt + 1, nk, wm, wn, lane, w, ld, NoHook{});
  }
  if (kt < kt_end) {
    stage_body<WN, NBJ, NSL, false, APLANE, 0, 0>(acc, ring, cur, nxt, kt, nk, wm, wn, lane, w, ld, NoHook{});
    ++kt;
  }
}

// K loop of nk stages over the slab loads `ld` (tiles of 256 x 32*WN*NBJ,
// NSL slabs in the ring). APLANE: the A tile is a plane operand.
// Start of a K loop of nsl >= 1 slabs: the loads of the first min(NSL, nsl)
// slabs and, with a prefetch, the first prefetch (slab NSL + 1); then the
// wait for slab 0.
template <int WN, int NBJ, int NSL, class SL>
__device__ __forceinline__ void ring_prologue(const SL &ld, Slab<WN, NBJ> *ring, int nsl, int w, int lane) {
  for (int sl = 0; sl < NSL && sl < nsl; ++sl) {
    const typename SL::Pre pre = ld.prep(sl);
#pragma unroll
    for (int j = 0; j < SL::N; ++j) ld.issue(pre, ring[sl], sl, w, lane, j);
  }
  if constexpr (SL::kPf) ld.prefetch((NSL + 1) < (nsl - 1) ? (NSL + 1) : (nsl - 1), w, lane);
  slab_wait<loads_per_slab<WN, NBJ>(), NSL - 1, SL::kPf ? 1 : 0>((nsl - 1) < (NSL - 1) ? (nsl - 1) : (NSL - 1));
}

template <int WN, int NBJ, int NSL, bool APLANE, class SL>
__device__ __forceinline__ void gemm_k(Acc<NBJ> &acc, Slab<WN, NBJ> *ring, const SL &ld, int nk) {
  const int lane = threadIdx.x & 63;
  const int w = wave_id(), wm = w & 1, wn = w >> 1;
  if (nk <= 0) return;
  const int nsl = (nk + 1) >> 1;
  ring_prologue<WN, NBJ, NSL>(ld, ring, nsl, w, lane);
  Frag<NBJ> cur, nxt;
  frag_read<WN, NBJ, APLANE>(cur, ring[0], 0, 0, wm, wn, lane);
  int kt = 0;
  stage_run<WN, NBJ, NSL, APLANE>(acc, ring, cur, nxt, kt, nk, nk, wm, wn, lane, w, ld);
}

// The wide GEMMs' loaders: 8 waves, 256 x 256 tiles.
using RmW = RmLoad<BM, 2 * WN_W>;
using CbW = CbLoad<BM, 2 * WN_W>;

// ---------------------------------------------------------------------------
// Up/gate GEMM with SwiGLU epilogue. i = token slot, j = interleaved W_ug row.
// Writes Z column-blocked [B][f/64][T_pad][64] and eta*Z^T in planes of 8 tokens [B][T_pad/8][f][8].
// grid: nx * ny workgroups, nx = 2f/256, ny = B*T_pad/256
struct A1Args {
  const bf16_t *x;
  const bf16_t *Wug;
  bf16_t *Z;
  bf16_t *ZT;
  float eta;
  int write_zt;
  int T, T_pad, d, f;
  int nx, ny;  // tiles along W_ug rows and along token slots
};

__global__ __launch_bounds__(NT_W, 1) void k_a1(A1Args p) {
  __shared__ __attribute__((aligned(16))) Slab<WN_W, NBJ_W> ring[NSL_W];
  int tx, ty;  // W_ug tile, token tile
  band_tile(xcd_tile(blockIdx.x, gridDim.x), p.nx, p.ny, 8, tx, ty);
  const int n0 = tx * 256;
  const int m0 = ty * BM;
  const int b = m0 / p.T_pad;
  const int pos0 = m0 - b * p.T_pad;
  SlabLoads<RmW, CbW> ld;
  ld.a.init(p.x + ((long long)b * p.T + pos0) * p.d, p.d, p.T - pos0, p.d, wave_id(), threadIdx.x & 63);
  ld.b.init(p.Wug + (long long)n0 * 64, 2LL * p.f * 64, 2 * p.f - n0, wave_id(), threadIdx.x & 63);
  Acc<NBJ_W> acc;
  acc_zero(acc);
  gemm_k<WN_W, NBJ_W, NSL_W, false>(acc, ring, ld, p.d / BK);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  bf16_t *ZTb = p.ZT + (long long)b * p.f * p.T_pad;
  // the wave's two 32-column blocks are a matching (up, gate) pair of W_ug rows
  const int feat = (n0 + wn * 64) / 2 + (lane & 31);
  if (feat < p.f) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const f32x16 &u = acc.v[bi][0];
      const f32x16 &g = acc.v[bi][1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pos = pos0 + wm * 128 + bi * 32 + 8 * q + 4 * (lane >> 5);
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = silu_fast(g[4 * q + r]) * u[4 * q + r];
        if (p.write_zt)
          store_nt(ZTb + ((long long)(pos >> 3) * p.f + feat) * 8 + (pos & 7), pack_bf16x2(p.eta * z[0], p.eta * z[1]),
                   pack_bf16x2(p.eta * z[2], p.eta * z[3]));
        bf16_t *zrow = p.Z + (((long long)b * (p.f / 64) + feat / 64) * p.T_pad + pos) * 64 + feat % 64;
#pragma unroll
        for (int r = 0; r < 4; ++r) store_nt(zrow + r * 64, f32_to_bf16(z[r]));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// General target rows V = U W_target (U: tap sums of the token embeddings),
// written straight into the layouts the scan reads: V^T K-blocked
// [B][T_pad/64][d][64] and, when clipping needs it, V row-major [B][T_pad][d].
// i = token slot, j = model dim a; the B operand is W_target^T [d][d] (row a
// holds column a of W_target). U rows past T are zero, so are those of V.
// grid: nx * ny workgroups, nx = d/256, ny = B*T_pad/256
struct TgtArgs {
  const bf16_t *U;
  const bf16_t *WtT;
  bf16_t *VT;
  bf16_t *Vrow;
  int T_pad, d, nx, ny;
};

__global__ __launch_bounds__(NT_W, 1) void k_target_gemm(TgtArgs p) {
  __shared__ __attribute__((aligned(16))) Slab<WN_W, NBJ_W> ring[NSL_W];
  int tx, ty;  // model-dim tile, token tile
  band_tile(xcd_tile(blockIdx.x, gridDim.x), p.nx, p.ny, 8, tx, ty);
  const int n0 = tx * 256;
  const int m0 = ty * BM;
  const int b = m0 / p.T_pad;
  const int pos0 = m0 - b * p.T_pad;
  SlabLoads<RmW, RmW> ld;
  ld.a.init(p.U + (long long)m0 * p.d, p.d, BM, p.d, wave_id(), threadIdx.x & 63);
  ld.b.init(p.WtT + (long long)n0 * p.d, p.d, 256, p.d, wave_id(), threadIdx.x & 63);
  Acc<NBJ_W> acc;
  acc_zero(acc);
  gemm_k<WN_W, NBJ_W, NSL_W, false>(acc, ring, ld, p.d / BK);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  bf16_t *VTb = p.VT + (long long)b * p.d * p.T_pad;
#pragma unroll
  for (int bj = 0; bj < NBJ_W; ++bj) {
    const int a = n0 + wn * WC_W + bj * 32 + (lane & 31);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pos = pos0 + wm * 128 + bi * 32 + 8 * q + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc.v[bi][bj][4 * q + r];
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(VTb + ((long long)(pos >> 6) * p.d + a) * 64 + (pos & 63)) = pk;
        if (p.Vrow) {
          bf16_t *vr = p.Vrow + ((long long)b * p.T_pad + pos) * p.d + a;
#pragma unroll
          for (int r = 0; r < 4; ++r) vr[(long long)r * p.d] = f32_to_bf16(v[r]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// State update with snapshots. i = hidden unit (ZT row), j = model dim (VT row),
// k = token slot. The fp32 accumulators ARE the state W[a][i] of one tile and
// stay in registers for the whole token stream; at each group start g*L the
// tile is written out as a bf16 snapshot.
//
// The state is cut into 256 x 256 tiles (i x a), numbered per sequence in
// bands of 8 along a (see band_tile) and then across sequences. Whole rounds
// of them (one per CU) run on the 8-wave configuration; a last partial round
// of at most 128 tiles is split into 256 x 128 halves that run as one round
// on the 4-wave configuration, so no CU idles for a whole round.

// Tile loads of the update with an L2 prefetch. Every eta Z^T tile is read by
// one XCD only, so its slabs come from HBM, one slab (two in the half-tile
// round) ahead of use without the prefetch. The workgroups that share an
// operand tile split its prefetch: the sa tiles (and halves) of a band of the
// tile order split the 256 lines of 128 bytes of an eta Z^T slab (8 planes of
// 32 lines), the sb tiles along x of an XCD's range split the BN rows (one
// line each) of a V^T slab. Waves 0 .. WN-1 touch the first share, waves WN ..
// 2WN-1 the second, each with one 4-byte DMA into a 256-byte LDS sink that
// nothing reads; each lane's offset within the slab is fixed at the start.
template <int WN, int BN>
struct UpdLoads : SlabLoads<PlLoad<2 * WN>, KbLoad<BN, 2 * WN>> {
  static constexpr bool kPf = true;
  uint32_t *sink;
  uint32_t vp;  // this lane's byte offset in the slab (A: plane and line, B: row)
  // sharer ka of sa takes lines [ka*256/sa, (ka+1)*256/sa) of the eta Z^T slab;
  // sharer kb of sb takes rows [kb*BN/sb, (kb+1)*BN/sb) of the V^T slab
  __device__ __forceinline__ void init_pf(uint32_t *sink_, int sa, int ka, int sb, int kb, int w, int lane) {
    sink = sink_;
    if (w < WN) {
      const int lo = ka * 256 / sa, n = (ka + 1) * 256 / sa - lo;
      const int per = (n + WN - 1) / WN < 64 ? (n + WN - 1) / WN : 64;
      int line = lo + w * per + lane % per;
      if (line > lo + n - 1) line = lo + n - 1;
      vp = (uint32_t)((line >> 5) * this->a.pstride * 2 + (line & 31) * 128);
    } else {
      const int lo = kb * BN / sb, n = (kb + 1) * BN / sb - lo;
      const int per = (n + WN - 1) / WN < 64 ? (n + WN - 1) / WN : 64;
      int row = lo + (w - WN) * per + lane % per;
      if (row > lo + n - 1) row = lo + n - 1;
      vp = (uint32_t)(row * 128);
    }
  }
  __device__ __forceinline__ void prefetch(int sl, int w, int lane) const {
    const __amdgpu_buffer_rsrc_t rs =
        w < WN ? __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(this->a.base + (long long)sl * 8 * this->a.pstride),
                                                   (short)0, 0x7fffffff, kBufferFlags)
               : __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(this->b.base + (long long)sl * this->b.kblk),
                                                   (short)0, 0x7fffffff, kBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)sink, 4, vp, 0, 0, 0);
  }
};

// LDS of the update: the ring and the prefetch sink in one object. (With the
// sink in an object of its own, the compiler cannot tell the prefetch DMA from
// the ring's, and waits for it before every fragment read.)
template <int WN, int NBJ, int NSL>
struct UpdLds {
  Slab<WN, NBJ> ring[NSL];
  uint32_t sink[64];
};

struct UpdArgs {
  const bf16_t *ZT;
  const bf16_t *VT;
  float *state;
  bf16_t *snap;
  int T_pad, kend, L, ngroups, d, f;
  int tile0;  // first 256 x 256 tile of this launch
};

// Write the accumulator tile as bf16 into a snapshot W[a][i], held as planes
// of 8 columns ([f/8][d][8]: element (a, i) at ((i/8)*d + a)*8 + i%8). Lane l
// holds, per group of 4 accumulator registers, four consecutive i of one a;
// lanes l and l+32 hold the two halves of one 16-byte chunk, and the 32 lanes
// of a half walk 32 consecutive a: each store instruction writes 512
// contiguous bytes. `lane_ptr` points at this lane's element for (bi, bj, q) =
// (0, 0, 0): a = j0 + wn*32*NBJ + l%32, i = i0 + wm*128 + 4*(l/32); tiles are
// always full (d, f multiples of 256).
template <int NBJ>
__device__ __forceinline__ void dump_snapshot(const Acc<NBJ> &acc, bf16_t *lane_ptr, int d) {
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj)
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 pk;
        pk.x = pack_bf16x2(acc.v[bi][bj][4 * q + 0], acc.v[bi][bj][4 * q + 1]);
        pk.y = pack_bf16x2(acc.v[bi][bj][4 * q + 2], acc.v[bi][bj][4 * q + 3]);
        *reinterpret_cast<uint2 *>(lane_ptr + (long long)(bi * 4 + q) * 8 * d + bj * 256) = pk;
      }
}

// WN = 4: workgroup n of the launch is tile tile0 + n (a 256 x 256 tile);
// WN = 2: workgroup n is half n%2 (128 columns of a) of tile tile0 + n/2.
template <int WN, int NBJ, int NSL>
__global__ __launch_bounds__(128 * WN, 1) void k_update(UpdArgs p) {
  __shared__ __attribute__((aligned(16))) UpdLds<WN, NBJ, NSL> lds;
  Slab<WN, NBJ> *ring = lds.ring;
  constexpr int BN = 32 * WN * NBJ;  // columns of a per workgroup
  const int nx = p.f / BM, ny = p.d / 256;
  const int n = xcd_tile(blockIdx.x, gridDim.x);
  const int t = p.tile0 + n / (256 / BN);
  const int b = t / (nx * ny);
  int tx, ty;
  band_tile(t - b * nx * ny, nx, ny, 8, tx, ty);
  const int i0 = tx * BM;
  const int j0 = ty * 256 + (n % (256 / BN)) * BN;
  const int lane = threadIdx.x & 63;
  const int w = wave_id(), wm = w & 1, wn = w >> 1;
  const long long df = (long long)p.d * p.f;
  // this lane's first element of the tile in the state ([d][f]) and in a snapshot ([f/8][d][8])
  const long long lane_off =
      (long long)(j0 + wn * 32 * NBJ + (lane & 31)) * p.f + i0 + wm * 128 + 4 * (lane >> 5);
  const long long lane_snap =
      (long long)((i0 + wm * 128) / 8) * 8 * p.d + (j0 + wn * 32 * NBJ + (lane & 31)) * 8 + 4 * (lane >> 5);
  float *st = p.state + b * df + lane_off;
  bf16_t *snap0 = p.snap + (long long)b * p.ngroups * df + lane_snap;

  Acc<NBJ> acc;
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
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

  // A: eta Z^T in planes of 8 tokens [T_pad/8][f][8]; B: V^T K-blocked [T_pad/64][d][64]
  UpdLoads<WN, BN> ld;
  ld.a.init(p.ZT + (long long)b * p.f * p.T_pad + (long long)i0 * 8, (long long)p.f * 8, lane);
  ld.b.init(p.VT + (long long)b * p.d * p.T_pad + (long long)j0 * 64, (long long)p.d * 64, w, lane);
  {
    // eta Z^T tile tx is shared by the tiles of its band (h of them) and their halves;
    // a V^T tile (or half) by the tiles along x of the XCD's range
    const int full = ny / 8, band = ty / 8, h = band < full ? 8 : ny - full * 8;
    const int halves = 256 / BN, half = n % halves;
    ld.init_pf(lds.sink, h * halves, (ty - band * 8) * halves + half, 16 / WN, tx % (16 / WN), w, lane);
  }
  const int nk = p.kend / BK;
  // Snapshot 0 is the entry state; group starts are multiples of the stage
  // depth, so snapshot g is written right after the last stage of group g-1,
  // while the following slabs are already in flight.
  dump_snapshot(acc, snap0, p.d);
  int g = 1;
  const int nsl = (nk + 1) >> 1;
  Frag<NBJ> cur, nxt;
  if (nk > 0) {
    ring_prologue<WN, NBJ, NSL>(ld, ring, nsl, w, lane);
    frag_read<WN, NBJ, true>(cur, ring[0], 0, 0, wm, wn, lane);
  }
  // The snapshot stores share the vector-memory counter with the tile loads.
  // The counted waits stay exact for the loads: loads complete in issue
  // order among themselves, so while a load is outstanding every later load
  // is too, and the count exceeds the number allowed; a store in flight can
  // only make a wait last longer.
  auto snapshot = [&](const Acc<NBJ> &a) {
    dump_snapshot(a, snap0 + (long long)g * df, p.d);
    ++g;
  };
  // Stages of group g-1 run plain; its last stage ends with snapshot g.
  // A group spans L/BK stages, an even number (L is a multiple of 64), so
  // every group ends on an odd stage.
  int kt = 0;
  for (; g < p.ngroups; ) {
    const int kt_last = g * (p.L / BK) - 1;  // last stage before group g starts
    stage_run<WN, NBJ, NSL, true>(acc, ring, cur, nxt, kt, kt_last, nk, wm, wn, lane, w, ld);
    pipelined_stage<WN, NBJ, NSL, true, true>(acc, ring, cur, nxt, kt, nk, wm, wn, lane, w, ld, snapshot);
    ++kt;
  }
  stage_run<WN, NBJ, NSL, true>(acc, ring, cur, nxt, kt, nk, nk, wm, wn, lane, w, ld);
#pragma unroll
  for (int bj = 0; bj < NBJ; ++bj) {
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
// same group. i = s, j = t; only tiles with i-tile <= j-tile that hold an
// unmasked entry are formed.
// grid: B * ngroups * nt(nt+1)/2 workgroups, nt = ceil(L/256)
constexpr int kMaxScorePairs = 136;  // the lower triangle of 16 x 16 tiles (L <= 4096)

struct ScoreArgs {
  const bf16_t *Z;
  bf16_t *P;
  float eta;
  int T, T_pad, L, C, ngroups, f, nt;
  // tiles (it, jt) of a full group that hold an unmasked entry; npairs = 0:
  // every tile of the lower triangle gets a workgroup (long groups)
  int npairs;
  unsigned char pit[kMaxScorePairs], pjt[kMaxScorePairs];
};

__global__ __launch_bounds__(NT_W, 1) void k_scores(ScoreArgs p) {
  __shared__ __attribute__((aligned(16))) Slab<WN_W, NBJ_W> ring[NSL_W];
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  int bg, it, jt;  // bg = b * ngroups + g
  if (p.npairs > 0) {
    bg = t / p.npairs;
    it = p.pit[t - bg * p.npairs];
    jt = p.pjt[t - bg * p.npairs];
  } else {
    const int ntri = p.nt * (p.nt + 1) / 2;
    bg = t / ntri;
    int u = t - bg * ntri;
    jt = 0;
    while (u > jt) u -= ++jt;  // u-th tile (it <= jt) of the lower triangle, jt-major
    it = u;
  }
  const int g = bg % p.ngroups, b = bg / p.ngroups;
  const long long gs = (long long)g * p.L;
  const int Lg = (int)((p.T - gs) < p.L ? (p.T - gs) : p.L);
  const int i0 = it * BM, j0 = jt * 256;
  if (j0 >= Lg) return;
  // A tile whose every s lies in the chunk of its last t or later is all
  // masked; the output GEMM never reads it (it stops before that chunk).
  const int jl = (j0 + 255 < Lg - 1) ? j0 + 255 : Lg - 1;
  if (i0 / p.C >= jl / p.C) return;
  const bf16_t *Zg = p.Z + ((long long)b * (p.f / 64) * p.T_pad + gs) * 64;  // Z column-blocked [f/64][T_pad][64]
  const long long zblk = (long long)p.T_pad * 64;
  SlabLoads<CbW, CbW> ld;
  ld.a.init(Zg + (long long)i0 * 64, zblk, (int)(p.T_pad - gs - i0), wave_id(), threadIdx.x & 63);
  ld.b.init(Zg + (long long)j0 * 64, zblk, (int)(p.T_pad - gs - j0), wave_id(), threadIdx.x & 63);
  Acc<NBJ_W> acc;
  acc_zero(acc);
  gemm_k<WN_W, NBJ_W, NSL_W, false>(acc, ring, ld, p.f / BK);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  bf16_t *Pg = p.P + ((long long)b * p.ngroups + g) * p.L * p.L;
#pragma unroll
  for (int bj = 0; bj < NBJ_W; ++bj) {
    const int t = j0 + wn * WC_W + bj * 32 + (lane & 31);
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
// Snapshot from an fp32 state with no update: snap[((i/8)*d + a)*8 + i%8] =
// bf16(state[a][i]). Thread (plane, a) converts one 8-column chunk.
__global__ __launch_bounds__(256) void k_state_to_snap(const float *state, bf16_t *snap, int d, int f) {
  const long long n = (long long)d * (f / 8);
  for (long long t = blockIdx.x * 256LL + threadIdx.x; t < n; t += (long long)gridDim.x * 256) {
    const int a = (int)(t % d);
    const long long pl = t / d;
    const float4 lo = *reinterpret_cast<const float4 *>(state + (long long)a * f + pl * 8);
    const float4 hi = *reinterpret_cast<const float4 *>(state + (long long)a * f + pl * 8 + 4);
    uint4 pk;
    pk.x = pack_bf16x2(lo.x, lo.y);
    pk.y = pack_bf16x2(lo.z, lo.w);
    pk.z = pack_bf16x2(hi.x, hi.y);
    pk.w = pack_bf16x2(hi.z, hi.w);
    *reinterpret_cast<uint4 *>(snap + t * 8) = pk;
  }
}

// ---------------------------------------------------------------------------
// Output GEMM: y[gL+t][a] = sum_k [snap | V^T][a][k] * [Z | P][t][k].
// i = a (model dim), j = t (token within group).
// grid: B * ngroups * (d/256) * ceil(L/256) workgroups
struct OutArgs {
  const bf16_t *Z;
  const bf16_t *P;
  const bf16_t *snap;
  const bf16_t *VT;
  bf16_t *y;
  int T, T_pad, L, C, ngroups, d, f, intra;
};

__global__ __launch_bounds__(NT_W, 1) void k_out(OutArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[kSmemOut / 2];
  Slab<WN_W, NBJ_W> *ring = reinterpret_cast<Slab<WN_W, NBJ_W> *>(smem);
  // one group's tiles are consecutive, token tiles fastest
  const int nx = p.d / BM, ny = (p.L + 255) / 256;
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int bg = t / (nx * ny), r = t - bg * nx * ny;
  const int i0 = (r / ny) * BM;
  const int j0 = (r % ny) * 256;
  const int b = bg / p.ngroups, g = bg % p.ngroups;
  const long long gs = (long long)g * p.L;
  const int Lg = (int)((p.T - gs) < p.L ? (p.T - gs) : p.L);
  if (j0 >= Lg) return;
  const int w8 = wave_id(), l8 = threadIdx.x & 63;
  Acc<NBJ_W> acc;
  acc_zero(acc);
  {  // segment 1: the group's snapshot ([f/8][d][8] planes) against Z, K = f
    SlabLoads<PlLoad<2 * WN_W>, CbW> ld;
    ld.a.init(p.snap + ((long long)b * p.ngroups + g) * p.d * p.f + (long long)i0 * 8, (long long)p.d * 8, l8);
    ld.b.init(p.Z + ((long long)b * (p.f / 64) * p.T_pad + gs + j0) * 64, (long long)p.T_pad * 64,
              (int)(p.T_pad - gs - j0), w8, l8);
    gemm_k<WN_W, NBJ_W, NSL_W, true>(acc, ring, ld, p.f / BK);
  }
  if (p.intra) {  // segment 2: V^T against P over the tokens before the last row's chunk
    const int jl = (j0 + 255 < Lg - 1) ? j0 + 255 : Lg - 1;
    const int kend = (jl / p.C) * p.C;  // start of the last row's chunk
    const int kv = (kend + 7) & ~7;
    const int nk2 = (kv + BK - 1) / BK;
    if (nk2 > 0) {
      // gs is a multiple of 64 (the plan's group length is), so V^T's slabs are whole blocks; columns of P
      // at or past kv read zero, so the V^T columns they meet contribute nothing
      SlabLoads<KbLoad<BM, 2 * WN_W>, RmLoad<BM, 2 * WN_W, true>> ld;
      ld.a.init(p.VT + (long long)b * p.d * p.T_pad + (gs >> 6) * ((long long)p.d * 64) + (long long)i0 * 64,
                (long long)p.d * 64, w8, l8);
      ld.b.init(p.P + ((long long)b * p.ngroups + g) * p.L * p.L + (long long)j0 * p.L, p.L, p.L - j0, kv, w8, l8);
      __syncthreads();  // every wave is done reading the ring before it is refilled
      gemm_k<WN_W, NBJ_W, NSL_W, false>(acc, ring, ld, nk2);
    }
  }

  // Epilogue through LDS ([token][model dim]) so y rows leave in whole lines.
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), wm = w & 1, wn = w >> 1;
  bf16_t *ly = smem;
  __syncthreads();  // every wave is done with the ring
#pragma unroll
  for (int bj = 0; bj < NBJ_W; ++bj) {
    const int tl = wn * WC_W + bj * 32 + (lane & 31);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int al = wm * 128 + bi * 32 + 8 * q + 4 * (lane >> 5);
        uint2 pk;
        pk.x = pack_bf16x2(acc.v[bi][bj][4 * q + 0], acc.v[bi][bj][4 * q + 1]);
        pk.y = pack_bf16x2(acc.v[bi][bj][4 * q + 2], acc.v[bi][bj][4 * q + 3]);
        *reinterpret_cast<uint2 *>(ly + tl * LY_P + al) = pk;
      }
  }
  __syncthreads();
  // 256 token rows x 512 bytes; rows past the group's end are not written
#pragma unroll
  for (int it = 0; it < 8192 / NT_W; ++it) {
    const int idx = it * NT_W + tid;
    const int tr = idx >> 5, ch = idx & 31;
    if (j0 + tr < Lg)
      *reinterpret_cast<uint4 *>(p.y + ((long long)b * p.T + gs + j0 + tr) * p.d + i0 + ch * 8) =
          *reinterpret_cast<const uint4 *>(ly + tr * LY_P + ch * 8);
  }
}

// ---------------------------------------------------------------------------
// Chunk Gram products for update clipping: ||V_i^T Z_i||_F^2 equals the sum of
// (V_i V_i^T) * (Z_i Z_i^T) over the chunk's token pairs. For s-tile u and
// t-tile w (256 tokens each) of one sequence, G_V = V_s V_t^T (K = d) is formed
// first and parked in a lane-private scratch (each lane later reads back only
// what it wrote), then G_Z = Z_s Z_t^T (K = f) in the same accumulators; the
// entries with s and t in the same chunk contribute G_V * G_Z, summed per row
// s (first over t 0..127, then 128..255) into rowpart[b][u][wr][s % 256]
// (wr = w - first t-tile that can share a chunk with the s-tile). Summing a
// chunk's rows over every wr gives its squared norm; the sums run in a fixed
// order, so results are deterministic.
// GATHER: V's rows are read from the target table through the ids (V[p] =
// E[ids[b][p+1]], zero for p >= T or an id outside [0, vocab)) instead of
// from a row-major copy.
// grid: B * (T_pad/256) * wspan workgroups of 512 threads
struct GramArgs {
  const bf16_t *Z;     // column-blocked [B][f/64][T_pad][64]
  const bf16_t *V;     // [B][T_pad][d], rows past T zero (without GATHER)
  const bf16_t *E;     // [vocab][d] (GATHER)
  const int32_t *ids;  // [B][T+1] (GATHER)
  float *gv;           // scratch: 256 KB per workgroup of the grid
  float *rowpart;      // [B][T_pad/256][wspan][256]
  int T, T_pad, C, d, f, wspan, vocab;
};

constexpr int GR_P = 129;  // fp32 pitch of a [256][128] product tile in LDS (conflict-free row sums)
constexpr int kSmemGram = cmax(kRingBytes, 256 * GR_P * 4);

template <bool GATHER>
__global__ __launch_bounds__(NT_W, 1) void k_chunk_gram(GramArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemGram];
  Slab<WN_W, NBJ_W> *ring = reinterpret_cast<Slab<WN_W, NBJ_W> *>(smem);
  const int nu = p.T_pad / 256;
  const int id = xcd_tile(blockIdx.x, gridDim.x);  // the t-tiles of an s-tile share an XCD
  const int wr = id % p.wspan;
  const int u = (id / p.wspan) % nu;
  const int b = id / (p.wspan * nu);
  const int s0 = u * 256;
  float *out = p.rowpart + (((long long)b * nu + u) * p.wspan + wr) * 256;
  const int s_last = (s0 + 255 < p.T - 1) ? s0 + 255 : p.T - 1;
  const int w = (int)((long long)(s0 / p.C) * p.C / 256) + wr;
  const long long w_end = (((long long)(s_last / p.C) + 1) * p.C - 1) / 256;
  const int w_hi = (int)(w_end < p.T_pad / 256 - 1 ? w_end : p.T_pad / 256 - 1);
  if (s0 >= p.T || w > w_hi) {  // no token pair of this tile shares a chunk
    if (threadIdx.x < 256) out[threadIdx.x] = 0.f;
    return;
  }
  const int t0 = w * 256;
  const int lane = threadIdx.x & 63, wv = wave_id(), wm = wv & 1, wn = wv >> 1;
  Acc<NBJ_W> acc;
  acc_zero(acc);
  if constexpr (GATHER) {
    SlabLoads<RmGather<BM, 2 * WN_W>, RmGather<BM, 2 * WN_W>> ld;
    const int32_t *tg = p.ids + (long long)b * (p.T + 1) + 1;  // target id of slot p at tg[p]
    ld.a.init(p.E, p.d, p.vocab, tg + s0, p.T - s0, wv, lane);
    ld.b.init(p.E, p.d, p.vocab, tg + t0, p.T - t0, wv, lane);
    gemm_k<WN_W, NBJ_W, NSL_W, false>(acc, ring, ld, p.d / BK);
  } else {
    const bf16_t *Vb = p.V + (long long)b * p.T_pad * p.d;
    SlabLoads<RmW, RmW> ld;
    ld.a.init(Vb + (long long)s0 * p.d, p.d, p.T_pad - s0, p.d, wv, lane);
    ld.b.init(Vb + (long long)t0 * p.d, p.d, p.T_pad - t0, p.d, wv, lane);
    gemm_k<WN_W, NBJ_W, NSL_W, false>(acc, ring, ld, p.d / BK);
  }
  // G_V to this lane's scratch: register group k (4 registers) at [k][lane]
  float4 *gv = reinterpret_cast<float4 *>(p.gv) + ((long long)id * 8 + wv) * (32 * 64) + lane;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < NBJ_W; ++bj)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        gv[((bi * NBJ_W + bj) * 4 + q) * 64] = make_float4(acc.v[bi][bj][4 * q], acc.v[bi][bj][4 * q + 1],
                                                           acc.v[bi][bj][4 * q + 2], acc.v[bi][bj][4 * q + 3]);
  __syncthreads();  // the second pass refills the ring
  acc_zero(acc);
  {
    const bf16_t *Zb = p.Z + (long long)b * (p.f / 64) * p.T_pad * 64;  // Z column-blocked [f/64][T_pad][64]
    SlabLoads<CbW, CbW> ld;
    ld.a.init(Zb + (long long)s0 * 64, (long long)p.T_pad * 64, p.T_pad - s0, wv, lane);
    ld.b.init(Zb + (long long)t0 * 64, (long long)p.T_pad * 64, p.T_pad - t0, wv, lane);
    gemm_k<WN_W, NBJ_W, NSL_W, false>(acc, ring, ld, p.f / BK);
  }
  // products of same-chunk pairs, in place of G_Z: row s0 + sl shares column
  // t's chunk when lo <= sl < lo + C (lo: the chunk's start less s0); one
  // 16-register group at a time, so few reloaded values are live at once
#pragma unroll
  for (int bj = 0; bj < NBJ_W; ++bj) {
    const int lo = (t0 + wn * WC_W + bj * 32 + (lane & 31)) / p.C * p.C - s0;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      pin();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 g = gv[((bi * NBJ_W + bj) * 4 + q) * 64];
        const float gq[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sl = wm * 128 + bi * 32 + 8 * q + 4 * (lane >> 5) + r;
          const float e = acc.v[bi][bj][4 * q + r];
          acc.v[bi][bj][4 * q + r] = (sl >= lo && sl < lo + p.C) ? e * gq[r] : 0.f;
        }
      }
    }
  }
  pin();
  // row sums through LDS, one 128-column half at a time
  float *tile = reinterpret_cast<float *>(smem);
  float sum = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // the ring, or the first half's tile, is no longer read
    if ((wn >> 1) == half) {
#pragma unroll
      for (int bj = 0; bj < NBJ_W; ++bj) {
        const int tl = (wn & 1) * WC_W + bj * 32 + (lane & 31);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            tile[(wm * 128 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * GR_P + tl] = acc.v[bi][bj][r];
      }
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      float part = 0.f;
      for (int t = 0; t < 128; ++t) part += tile[threadIdx.x * GR_P + t];
      sum = half == 0 ? part : sum + part;
    }
  }
  if (threadIdx.x < 256) out[threadIdx.x] = sum;
}

// ---------------------------------------------------------------------------
// Target gather, transposed and K-blocked: V^T[b][p/64][a][p%64] = E[ids[b][p+1]][a].
// A 64-slot x 64-feature tile passes through LDS so both the row reads of E and
// the writes (one contiguous 8 KB block) are 16 B per lane. With Vrow non-null
// the rows are also written row-major, Vrow[b][p][a] (used by update clipping).
// With cfac non-null, slot p is scaled by the clipping factor cfac[b][p/C]
// (bf16 -> fp32, times the factor, rounded to bf16).
// grid: (T_pad/64, d/64, B)
__global__ __launch_bounds__(256) void k_gather_vt(const int32_t *ids, const bf16_t *E, int vocab, bf16_t *VT,
                                                   bf16_t *Vrow, const float *cfac, int C, int nchunks, int T,
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
    if (cfac && pos < T) {
      const float c = cfac[(long long)b * nchunks + pos / C];
      bf16_t *e = reinterpret_cast<bf16_t *>(&v);
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = f32_to_bf16(bf16_to_f32(e[k]) * c);
    }
    // 16-byte column groups XOR-swizzled by (row / 8) % 8: the transposing
    // reads below take one column from rows 8 apart, which the plain layout
    // puts in the same banks
    *reinterpret_cast<uint4 *>(&tile[pl][(seg ^ ((pl >> 3) & 7)) * 8]) = v;
    if (Vrow) *reinterpret_cast<uint4 *>(Vrow + ((long long)b * T_pad + pos) * d + a0 + seg * 8) = v;
  }
  __syncthreads();
  bf16_t *blk = VT + ((long long)b * (T_pad / 64) + blockIdx.x) * d * 64;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int al = pass * 32 + (tid >> 3);
    const int ax = al ^ (seg << 3);  // rows seg*8 .. seg*8+7 carry the swizzle seg
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wv[e] = (uint32_t)tile[seg * 8 + 2 * e][ax] | ((uint32_t)tile[seg * 8 + 2 * e + 1][ax] << 16);
    *reinterpret_cast<uint4 *>(blk + (long long)(a0 + al) * 64 + seg * 8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

}  // namespace

hipError_t launch_gather_vt_bf16(const int32_t *ids, const bf16_t *E, int vocab, bf16_t *VT, bf16_t *Vrow,
                                 const float *cfac, const Layout &lay, hipStream_t s) {
  dim3 grid(lay.T_pad / 64, lay.d / 64, lay.B);
  const int nchunks = (int)((lay.T + (long long)lay.C - 1) / lay.C);
  hipLaunchKernelGGL(k_gather_vt, grid, dim3(256), 0, s, ids, E, vocab, VT, Vrow, cfac, lay.C, nchunks, lay.T,
                     lay.T_pad, lay.d);
  return hipGetLastError();
}

hipError_t launch_chunk_gram_bf16(const bf16_t *Z, const bf16_t *Vrow, const bf16_t *E, const int32_t *ids, int vocab,
                                  float *gv, float *rowpart, int wspan, const Layout &lay, hipStream_t s) {
  const long long n = (long long)lay.B * (lay.T_pad / 256) * wspan;
  if (n >= (1LL << 31) / 8) return hipErrorInvalidConfiguration;
  if (!Vrow && (long long)vocab * lay.d * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  GramArgs p{Z, Vrow, E, ids, gv, rowpart, lay.T, lay.T_pad, lay.C, lay.d, lay.f, wspan, vocab};
  if (Vrow)
    hipLaunchKernelGGL(k_chunk_gram<false>, dim3((unsigned)n), dim3(NT_W), 0, s, p);
  else
    hipLaunchKernelGGL(k_chunk_gram<true>, dim3((unsigned)n), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_a1_bf16(const bf16_t *x, const bf16_t *Wug, bf16_t *Z, bf16_t *ZT, float eta, int write_zt,
                          const Layout &lay, hipStream_t s) {
  const int nx = (2 * lay.f + 255) / 256;
  const long long ny = (long long)lay.B * lay.T_pad / BM;
  if (nx * ny >= (1LL << 31)) return hipErrorInvalidConfiguration;
  A1Args p{x, Wug, Z, ZT, eta, write_zt, lay.T, lay.T_pad, lay.d, lay.f, nx, (int)ny};
  hipLaunchKernelGGL(k_a1, dim3((unsigned)(nx * ny)), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_target_gemm_bf16(const bf16_t *U, const bf16_t *WtT, bf16_t *VT, bf16_t *Vrow, const Layout &lay,
                                  hipStream_t s) {
  const int nx = lay.d / 256;
  const long long ny = (long long)lay.B * lay.T_pad / BM;
  if (nx * ny >= (1LL << 31)) return hipErrorInvalidConfiguration;
  TgtArgs p{U, WtT, VT, Vrow, lay.T_pad, lay.d, nx, (int)ny};
  hipLaunchKernelGGL(k_target_gemm, dim3((unsigned)(nx * ny)), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_update_bf16(const bf16_t *ZT, const bf16_t *VT, float *state, bf16_t *snap, const Layout &lay,
                              hipStream_t s) {
  const int kend = (int)round_up_ll(lay.T, BK);
  const long long tiles = (long long)lay.B * (lay.f / BM) * (lay.d / 256);
  if (tiles * 2 >= (1LL << 31)) return hipErrorInvalidConfiguration;
  // whole rounds on the wide configuration, a last round of <= 128 tiles as halves
  const int cus = 256;
  const long long rem = tiles % cus;
  const long long whole = rem <= cus / 2 ? tiles - rem : tiles;
  UpdArgs p{ZT, VT, state, snap, lay.T_pad, kend, lay.L, lay.ngroups, lay.d, lay.f, 0};
  if (whole > 0) hipLaunchKernelGGL((k_update<WN_W, NBJ_W, NSL_W>), dim3((unsigned)whole), dim3(NT_W), 0, s, p);
  if (tiles > whole) {
    p.tile0 = (int)whole;
    hipLaunchKernelGGL((k_update<WN_U, NBJ_U, NSL_U>), dim3((unsigned)(2 * (tiles - whole))), dim3(NT_U), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_scores_bf16(const bf16_t *Z, bf16_t *P, float eta, const Layout &lay, hipStream_t s) {
  const int nt = (lay.L + 255) / 256;
  ScoreArgs p{Z, P, eta, lay.T, lay.T_pad, lay.L, lay.C, lay.ngroups, lay.f, nt, 0, {}, {}};
  if (nt * (nt + 1) / 2 <= kMaxScorePairs) {
    // the tiles of a full group that the kernel would not skip, jt-major
    for (int jt = 0; jt < nt; ++jt) {
      const int jl = (jt * 256 + 255 < lay.L - 1) ? jt * 256 + 255 : lay.L - 1;
      for (int it = 0; it <= jt; ++it)
        if (it * 256 / lay.C < jl / lay.C) {
          p.pit[p.npairs] = (unsigned char)it;
          p.pjt[p.npairs] = (unsigned char)jt;
          ++p.npairs;
        }
    }
    if (p.npairs == 0) return hipSuccess;  // one chunk per group: no within-group term
  }
  const long long n = (long long)lay.B * lay.ngroups * (p.npairs > 0 ? p.npairs : nt * (nt + 1) / 2);
  if (n >= (1LL << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_scores, dim3((unsigned)n), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_state_to_snap_bf16(const float *state, bf16_t *snap, int d, int f, hipStream_t s) {
  if (d <= 0 || f <= 0 || f % 8) return hipErrorInvalidValue;
  const long long n = (long long)d * (f / 8);
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_state_to_snap, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s, state, snap, d,
                     f);
  return hipGetLastError();
}

hipError_t launch_out_bf16(const bf16_t *Z, const bf16_t *P, const bf16_t *snap, const bf16_t *VT, bf16_t *y,
                           const Layout &lay, hipStream_t s) {
  OutArgs p{Z, P, snap, VT, y, lay.T, lay.T_pad, lay.L, lay.C, lay.ngroups, lay.d, lay.f, lay.intra};
  const long long n = (long long)lay.B * lay.ngroups * (lay.d / BM) * ((lay.L + 255) / 256);
  if (n >= (1LL << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_out, dim3((unsigned)n), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}
