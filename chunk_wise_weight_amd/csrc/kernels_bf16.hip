// bf16 MFMA kernels of the chunk-wise fast-weight path (gfx950).
//
// Every contraction is written as D[i][j] = sum_k A[i][k] * B[j][k] with both
// operands K-contiguous ("NT" form). A block has 2 x WN waves; each wave
// computes 128 x (32*NBJ) with v_mfma_f32_16x16x32_bf16 and fp32 accumulators.
// Under the chip's power limit the 16x16x32 form runs at a higher clock than
// the 32x32x16 one (measured with MFMAs alone on every CU: 2.0 against
// 1.73 GHz), at the same work per cycle. Every GEMM uses 8 waves (WN = 4, NBJ = 2: 256 x 256 tiles, two
// waves per SIMD so one can issue MFMAs while the other waits), except the
// last, partial round of the state update, which runs 256 x 128 halves on 4
// waves (WN = 2, NBJ = 2).
//
// Tiles go from HBM straight into LDS with 16-byte buffer loads (no register
// staging) in slabs of 64 columns, so that every row contributes one whole
// 128-byte line: whole lines fill LDS at twice the rate of half lines. A ring
// of NSL slabs keeps the next slabs in flight while one is multiplied, and
// each wave waits only for the oldest slab it needs. The MFMAs run in stages
// of 32 (two per slab), one MFMA per 16 x 16 output tile; within a stage the
// fragment reads of its second half of rows and of the next stage are issued
// behind MFMAs already queued (a software pipeline). The eight 16-byte chunks of each 128-byte LDS row are
// XOR-swizzled so that the fragment reads are free of bank conflicts. Rows or
// columns outside an operand's valid range are fetched through an
// out-of-range buffer offset, which the hardware returns as zero.
//
// Operands are row-major (element (r, k) at r*ld + k), K-blocked by 64
// (element (r, k) at (k/64)*kblk + r*64 + k%64), or held in planes of 8
// columns (element (r, k) at (k/8)*pstride + r*8 + k%8). V^T and Z are
// K-blocked (Z's blocks hold every token slot, [f/64][S][64]), so one slab
// of a tile is one contiguous block instead of rows strided by the whole
// stream length or by f. The state update, whose contraction runs over the
// tokens, takes Z's blocks as they are and reads its fragments with
// transposing LDS reads. The snapshots are planes: the MFMA register layout
// holds four consecutive i of one j per lane, so a store instruction of 16
// columns x 16 bytes is 256 contiguous bytes in a plane (in row-major or
// K-blocked form it would touch 16 lines); a plane slab loads as 1 KB
// contiguous pieces into an LDS tile of [8][256][8], whose fragment reads
// need no swizzle.
//
// MFMA 16x16x32 register layout (lane l, accumulator register r):
//   A operand: row i = l % 16, k = 8*(l/16) .. +7;  B operand: column j = l % 16, same k.
//   D: j = l % 16, i = 4*(l/16) + r.
// So each lane holds, per accumulator (a group of 4 registers), four
// consecutive i for one j: epilogues store 4 consecutive elements along i.
// A wave's accumulator (gi, gj), gi < 8, gj < 2*NBJ, covers rows
// 16 gi .. +15 and columns 16 gj .. +15 of its 128 x (32*NBJ) sub-tile.
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
  f32x4 v[8][2 * NBJ];
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

// Chunk swizzle of the kAZ tile (below): k row r holds logical chunk c at
// c ^ zsw(r). A transposing read of one 16-lane group g covers 4 consecutive
// k rows r0 + 8g .. +3 and one pair of adjacent chunks in each; the LDS
// serves 32 lanes (two groups, 8 rows apart) at a time. zsw(r) =
// 2*((r%4) ^ (r/8 % 2)) gives the 4 rows of one parity (rows of a 128-byte
// stride alternate between the two halves of the 64 banks) of the two groups
// the four disjoint chunk pairs of that half, so the read is free of bank
// conflicts.
__device__ __forceinline__ int zsw(int r) { return ((r & 3) ^ ((r >> 3) & 1)) << 1; }

template <int NBJ>
__device__ __forceinline__ void acc_zero(Acc<NBJ> &acc) {
#pragma unroll
  for (int gi = 0; gi < 8; ++gi)
#pragma unroll
    for (int gj = 0; gj < 2 * NBJ; ++gj)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc.v[gi][gj][r] = 0.f;
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

// LDS DMA issued as an instruction the compiler does not track (the state
// update's loads). The compiler treats a tracked LDS DMA as a pending write to
// LDS, and before a transposing read (ds_read_b64_tr_b16) it cannot tell that
// the read's buffer is not the one in flight, so it waits for every DMA: the
// ring's lookahead would be lost once per slab. Untracked, the loads are
// ordered by the kernel's own counted waits and barriers alone (slab_wait),
// which is how the ring is built anyway. No register outputs: the data goes
// to LDS at M0 + 16 (4) bytes per lane. M0 is the compiler's register: the
// block saves it in a scalar register of its own and puts it back.
__device__ __forceinline__ void dma16_untracked(__amdgpu_buffer_rsrc_t rs, void *lds, uint32_t voff, uint32_t soff) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)lds);
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(base), "v"(voff), "s"(rs), "s"(soff)
      : "memory");
}
__device__ __forceinline__ void dma4_untracked(__amdgpu_buffer_rsrc_t rs, void *lds, uint32_t voff, uint32_t soff) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)lds);
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(base), "v"(voff), "s"(rs), "s"(soff)
      : "memory");
}

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
// gap: tile rows 128 and up come from operand rows r + gap (two 128-row
// pieces of one operand in one tile).
template <int ROWS, int NW>
struct CbLoad {
  static constexpr int WR = ROWS / NW, N = WR / 8;
  const bf16_t *base;
  long long kblk;
  int bytes;
  // a fixed bound: with vo[N] here, the host pass of hipcc rejects SlabLoads<PlLoad, CbLoad>
  uint32_t vo[8];
  static_assert(N <= 8, "lane offsets per wave");
  __device__ __forceinline__ void init(const bf16_t *base_, long long kblk_, int nrows, int w, int lane,
                                       int gap = 0) {
    base = base_;
    kblk = kblk_;
    const long long by = (long long)(nrows > 0 ? nrows : 0) * 128;
    bytes = (int)(by < 0x7fffffffLL ? by : 0x7fffffffLL);
    const int lr = lane >> 3;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int row = w * WR + 8 * n + lr;
      vo[n] = (uint32_t)((row + (row >= 128 ? gap : 0)) * 128 + (((lane & 7) ^ swz(row)) << 4));
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
  // the same load, untracked (dma16_untracked)
  __device__ __forceinline__ void issue_untracked(const Pre &rs, bf16_t *tile, int w, int n) const {
    dma16_untracked(rs, tile + (w * WR + 8 * n) * SK, (n & 1) ? vd : ve, (w * WR + 8 * n) * 128);
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

// Z blocks as the A tile of the state update (kAZ): tile rows i are 256
// hidden units (4 blocks of 64 of Z, [f/64][S][64]), k the token slots. The
// slab of block b is 64 slots x 128 bytes, contiguous in memory, and lands as
// LDS rows k of [4][64][64] with chunk swizzle zsw. Wave w of NW loads 8N of
// the 64 rows of block w/(NW/4), 8 rows (1 KB) per load; lane l fills row
// 8n + l/8 of its share, physical chunk l%8 = logical chunk (l%8) ^ zsw(row).
// The swizzle depends on n only through its parity (the share starts at a
// multiple of 8), so two lane offsets serve every load. Every slot of a slab
// exists in Z (slabs stay within the sequence's padded slots).
template <int NW>
struct ZbLoad {
  static constexpr int N = 32 / NW;  // loads per wave per slab
  static constexpr int WB = NW / 4;  // waves per block
  const bf16_t *base;                // this wave's block at the tile's first slot
  int r0;                            // this wave's first row in its block
  int blk;                           // this wave's block
  uint32_t ve, vd;                   // lane offsets for even / odd n
  __device__ __forceinline__ void init(const bf16_t *Z, long long S, int i0, long long slot0, int w, int lane) {
    blk = w / WB;
    r0 = (w % WB) * 8 * N;
    base = Z + ((long long)(i0 / 64 + blk) * S + slot0) * 64;
    const int r = r0 + (lane >> 3);
    ve = (uint32_t)(r * 128 + (((lane & 7) ^ zsw(r)) << 4));
    vd = (uint32_t)(r * 128 + (((lane & 7) ^ zsw(r + 8)) << 4));
  }
  using Pre = __amdgpu_buffer_rsrc_t;
  __device__ __forceinline__ Pre prep(int sl) const {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(base + (long long)sl * 64 * 64), (short)0,
                                             0x7fffffff, kBufferFlags);
  }
  __device__ __forceinline__ void issue(const Pre &rs, bf16_t *tile, int, int, int, int n) const {
    dma16_untracked(rs, tile + (blk * 64 + r0 + 8 * n) * 64, (n & 1) ? vd : ve, n * 1024);
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

// MFMA fragments of a 32-deep stage: the A fragments of the wave's rows
// 0-63 (lo) and 64-127 (hi), 16 rows each, and two sets of B fragments (16
// columns each), set s used by the stages of parity s, so that the next
// stage's set can load while this stage's last MFMAs still read theirs.
template <int NBJ>
struct Frag {
  bf16x8 lo[4], hi[4];
  bf16x8 b[2][2 * NBJ];
};

// How the A tile of a slab is held in LDS:
//   kARows:   256 rows of 64 k, 16-byte chunks swizzled by swz (see lds_off);
//   kAPlanes: 8 planes of [256 rows][8 k] (chunk c of row r at (c*256 + r)*8);
//   kAZ:      Z blocks: [4][64 k][64 rows] (row i of the tile is column i%64
//             of block i/64: the tile is held transposed), 16-byte chunks of
//             each k row swizzled by zsw. The fragments come from transposing
//             reads.
constexpr int kARows = 0, kAPlanes = 1, kAZ = 2;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// A fragment of a kAZ tile: rows 16gi + l%16 of a 64-row block (lane l), k
// 8(l/16) .. +7 of the stage, from two transposing reads (ds_read_b64_tr_b16)
// of 4 k rows each. In each 16-lane group g, lane t addresses k row
// 8g + t/4 (+4 for the second read), columns 4(t%4) .. +3 of the fragment's
// 16 (one 8-byte piece), and receives column t of the 4 rows. This is lane
// l's element offset for gi = 0; the chunk pair of fragment gi is gi
// further on, which in the swizzled row is `^ (gi << 4)` (zsw is even, so
// the XOR leaves the 8-byte half within the chunk alone).
__device__ __forceinline__ int az_lane_off(int lane) {
  const int t = lane & 15, g = lane >> 4;
  const int krow = 8 * g + (t >> 2);
  const int chunk = ((t & 3) >> 1) ^ zsw(krow);
  return krow * 64 + chunk * 8 + 4 * (t & 1);
}

// The A fragments of rows 64hf .. 64hf+63 of the wave's 128 (hf = 0, 1) for
// stage half h (0 or 1) of an LDS slab.
template <int WN, int NBJ, int AMODE = kARows>
__device__ __forceinline__ void read_a(bf16x8 (&a)[4], const Slab<WN, NBJ> &st, int h, int hf, int wm, int lane) {
  const int c = 4 * h + (lane >> 4);
  if constexpr (AMODE == kAZ) {
    const int lo = az_lane_off(lane);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const bf16_t *pa = st.a + (wm * 2 + hf) * 4096 + h * 2048 + (lo ^ (gi << 4));
      const bf16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(pa));
      const bf16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(pa + 256));
      a[gi] = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  } else {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int r = wm * 128 + hf * 64 + gi * 16 + (lane & 15);
      a[gi] = *reinterpret_cast<const bf16x8 *>(st.a + (AMODE == kAPlanes ? (c * BM + r) * 8 : lds_off(r, c)));
    }
  }
}

// The B fragments of the wave's 32*NBJ columns for stage half h of a slab.
template <int WN, int NBJ>
__device__ __forceinline__ void read_b(bf16x8 (&b)[2 * NBJ], const Slab<WN, NBJ> &st, int h, int wn, int lane) {
  const int c = 4 * h + (lane >> 4);
#pragma unroll
  for (int gj = 0; gj < 2 * NBJ; ++gj)
    b[gj] = *reinterpret_cast<const bf16x8 *>(st.b + lds_off(wn * 32 * NBJ + gj * 16 + (lane & 15), c));
}

// The MFMAs of row fragment GI (0..7) of a stage.
template <int GI, int NBJ>
__device__ __forceinline__ void frag_mma(Acc<NBJ> &acc, const bf16x8 &a, const bf16x8 (&b)[2 * NBJ]) {
#pragma unroll
  for (int gj = 0; gj < 2 * NBJ; ++gj)
    acc.v[GI][gj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[gj], acc.v[GI][gj], 0, 0, 0);
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
// entry fr.lo and fr.b[kt%2] hold (or are loading) stage kt's fragments of
// rows 0-63 and of the columns; on exit fr.lo and fr.b[(kt+1)%2] hold those
// of stage kt+1. Every LDS read and tile-load issue sits behind MFMAs already
// queued, so the matrix cores keep running while they wait:
//   read rows 64-127 of kt -> fr.hi | MFMAs of row fragment 0
//   at the end of a slab: wait for the next slab + barrier
//   MFMAs of row fragments 1-7, with this wave's loads of slab kt/2 + NSL
//   (into the buffer just finished) issued between them, and rows 0-63 and
//   the columns of kt+1 read after fragment 4 (fr.lo is no longer read).
// After the barrier no wave reads the finished slab's buffer again (all its
// reads were issued before, and the wait includes lgkmcnt(0)), so it can be
// refilled. Spreading the loads keeps a burst of them from stalling the MFMA
// issue. With AFTER, after_fn(acc) runs once all of stage kt's MFMAs are
// queued, and the next fragments are read only then (few registers live).
// Loads with a prefetch (SL::kPf) also touch, in every odd stage, this
// workgroup's share of slab kt/2 + NSL + 2, so that the slab's own loads two
// stages later find it in L2.
// H (= kt % 2) is fixed at compile time (it picks the B fragment set), and so
// is REFILL (this stage refills the buffer it finished: 1/0) where the caller
// knows it, else -1 (decided here at run time).
// sc is the ring buffer of slab kt/2, sn that of the slab after it.
template <int WN, int NBJ, int NSL, bool AFTER, int AMODE, int H, int REFILL, class SL, class AfterFn>
__device__ __forceinline__ void stage_body(Acc<NBJ> &acc, Slab<WN, NBJ> &sc, Slab<WN, NBJ> &sn, Frag<NBJ> &fr, int kt,
                                           int nk, int wm, int wn, int lane, int w, const SL &ld,
                                           AfterFn &&after_fn) {
  constexpr int LPS = loads_per_slab<WN, NBJ>();
  static_assert(SL::N == LPS, "the slab loads match the tile configuration");
  static_assert(H == 0 || H == 1, "the stage parity is known at compile time");
  constexpr int h = H;
  const int sl = kt >> 1;
  const int nsl = (nk + 1) >> 1;
  const bool refill = REFILL >= 0 ? REFILL == 1 : (h == 1 && sl + NSL < nsl);
  const bf16x8(&b)[2 * NBJ] = fr.b[h];
  // rows 0-63 and the columns of stage kt+1: the next slab's buffer after an odd stage
  auto read_next = [&]() {
    if constexpr (h == 1) {
      read_a<WN, NBJ, AMODE>(fr.lo, sn, 0, 0, wm, lane);
      read_b<WN, NBJ>(fr.b[0], sn, 0, wn, lane);
    } else {
      read_a<WN, NBJ, AMODE>(fr.lo, sc, 1, 0, wm, lane);
      read_b<WN, NBJ>(fr.b[1], sc, 1, wn, lane);
    }
  };
  read_a<WN, NBJ, AMODE>(fr.hi, sc, h, 1, wm, lane);
  pin();
  frag_mma<0>(acc, fr.lo[0], b);
  pin();
  const bool more = kt + 1 < nk;  // always true when refilling
  if (h == 1 && (refill || more)) {
    const int later = (nsl - 2 - sl) < (NSL - 2) ? (nsl - 2 - sl) : (NSL - 2);
    slab_wait<LPS, NSL - 2, SL::kPf ? 1 : 0>(later);
  }
  const int rs = sl + NSL;
  Slab<WN, NBJ> &dst = sc;  // the buffer just finished refills with slab rs
  typename SL::Pre pre{};
  if (refill) pre = ld.prep(rs);
  pin();
  frag_mma<1>(acc, fr.lo[1], b);
  if (refill) issue_point<LPS, 0>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<2>(acc, fr.lo[2], b);
  if (refill) issue_point<LPS, 1>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<3>(acc, fr.lo[3], b);
  if (refill) issue_point<LPS, 2>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<4>(acc, fr.hi[0], b);
  pin();
  // unconditional (past the end it reads a stale buffer of the ring): no
  // branch, so the compiler can count the reads and wait for each exactly
  if (!AFTER) read_next();
  if (refill) issue_point<LPS, 3>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<5>(acc, fr.hi[1], b);
  if (refill) issue_point<LPS, 4>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<6>(acc, fr.hi[2], b);
  if (refill) issue_point<LPS, 5>(ld, pre, dst, rs, w, lane);
  pin();
  frag_mma<7>(acc, fr.hi[3], b);
  if (refill) issue_point<LPS, 6>(ld, pre, dst, rs, w, lane);
  // one prefetch per odd stage, always issued, so every slab wait counts one
  if constexpr (SL::kPf) {
    if (h == 1) ld.prefetch((sl + NSL + 2) < (nsl - 1) ? (sl + NSL + 2) : (nsl - 1), w);
  }
  pin();
  if (AFTER) {
    after_fn(acc);
    read_next();
    pin();
  }
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

// The same within each round of R workgroups (R: the workgroups resident at
// once, one per CU, in launch order): round r's workgroups take logical tiles
// r*R .. r*R + R - 1, XCD k a contiguous range of them. Where the logical order
// keeps tiles that share operands together (the state update's tiles of one
// sequence, the output's and the scores' tiles of one group), the whole chip
// then works on one stretch of it at a time, and the XCDs share the slabs of
// the stretch in the MALL; with xcd_tile alone, the 8 XCDs would walk 8
// distant stretches (8 different documents of a packed call, 8 groups 16
// apart in the output of a 128-group stream).
__device__ __forceinline__ int xcd_tile_rounds(int n, int N, int R) {
  const int r0 = n / R * R;
  const int Rn = N - r0 < R ? N - r0 : R;
  return r0 + xcd_tile(n - r0, Rn);
}

// R for the kernels of one workgroup per CU: the compute units, rounded down
// to a multiple of the XCD count (at least one per XCD).
static int launch_round(int cus) { return cus >= kXcds ? cus / kXcds * kXcds : kXcds; }

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
// count of stages ends on a lone even stage. Leaves kt = kt_end. `pair(kt,
// refill)` runs the two stages of slab kt/2 (refill: whether the second one
// refills), `lone(kt)` a lone even stage.
template <int NSL, class Pair, class Lone>
__device__ __forceinline__ void stage_phases(int &kt, int kt_end, int nk, Pair &&pair, Lone &&lone) {
  const int nsl = (nk + 1) >> 1;
  const int kref = nsl > NSL ? 2 * (nsl - NSL) : 0;  // first stage past the refilling slabs
  const int k1 = kref < kt_end ? kref : kt_end;
  for (; kt + 1 < k1; kt += 2) pair(kt, std::true_type{});
  for (; kt + 1 < kt_end; kt += 2) pair(kt, std::false_type{});
  if (kt < kt_end) {
    lone(kt);
    ++kt;
  }
}

// The ring as one LDS array: buffer cb (runtime) holds slab kt/2.
template <int WN, int NBJ, int NSL, int AMODE, class SL>
__device__ __forceinline__ void stage_run(Acc<NBJ> &acc, Slab<WN, NBJ> *ring, Frag<NBJ> &fr, int &kt, int &cb,
                                          int kt_end, int nk, int wm, int wn, int lane, int w, const SL &ld) {
  stage_phases<NSL>(
      kt, kt_end, nk,
      [&](int k, auto refill) {
        const int nb = cb + 1 == NSL ? 0 : cb + 1;
        stage_body<WN, NBJ, NSL, false, AMODE, 0, 0>(acc, ring[cb], ring[nb], fr, k, nk, wm, wn, lane, w, ld,
                                                     NoHook{});
        stage_body<WN, NBJ, NSL, false, AMODE, 1, decltype(refill)::value ? 1 : 0>(
            acc, ring[cb], ring[nb], fr, k + 1, nk, wm, wn, lane, w, ld, NoHook{});
        cb = nb;
      },
      [&](int k) {
        const int nb = cb + 1 == NSL ? 0 : cb + 1;
        stage_body<WN, NBJ, NSL, false, AMODE, 0, 0>(acc, ring[cb], ring[nb], fr, k, nk, wm, wn, lane, w, ld,
                                                     NoHook{});
      });
}

// K loop of nk stages over the slab loads `ld` (tiles of 256 x 32*WN*NBJ,
// NSL slabs in the ring). AMODE: how the A tile is held (kARows, kAPlanes, kAZ).
// Start of a K loop of nsl >= 1 slabs: the loads of the first min(NSL, nsl)
// slabs and, with a prefetch, the first prefetch (slab NSL + 1); then the
// wait for slab 0. buf(sl) is the ring buffer of slab sl < NSL.
template <int WN, int NBJ, int NSL, class SL, class Buf>
__device__ __forceinline__ void ring_prologue(const SL &ld, Buf &&buf, int nsl, int w, int lane) {
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    if (sl < nsl) {
      const typename SL::Pre pre = ld.prep(sl);
#pragma unroll
      for (int j = 0; j < SL::N; ++j) ld.issue(pre, buf(sl), sl, w, lane, j);
    }
  }
  if constexpr (SL::kPf) ld.prefetch((NSL + 1) < (nsl - 1) ? (NSL + 1) : (nsl - 1), w);
  slab_wait<loads_per_slab<WN, NBJ>(), NSL - 1, SL::kPf ? 1 : 0>((nsl - 1) < (NSL - 1) ? (nsl - 1) : (NSL - 1));
}

template <int WN, int NBJ, int NSL, int AMODE, class SL>
__device__ __forceinline__ void gemm_k(Acc<NBJ> &acc, Slab<WN, NBJ> *ring, const SL &ld, int nk) {
  const int lane = threadIdx.x & 63;
  const int w = wave_id(), wm = w & 1, wn = w >> 1;
  if (nk <= 0) return;
  const int nsl = (nk + 1) >> 1;
  ring_prologue<WN, NBJ, NSL>(ld, [&](int sl) -> Slab<WN, NBJ> & { return ring[sl]; }, nsl, w, lane);
  Frag<NBJ> fr;
  read_a<WN, NBJ, AMODE>(fr.lo, ring[0], 0, 0, wm, lane);
  read_b<WN, NBJ>(fr.b[0], ring[0], 0, wn, lane);
  int kt = 0, cb = 0;
  stage_run<WN, NBJ, NSL, AMODE>(acc, ring, fr, kt, cb, nk, nk, wm, wn, lane, w, ld);
}

// The wide GEMMs' loaders: 8 waves, 256 x 256 tiles.
using RmW = RmLoad<BM, 2 * WN_W>;
using CbW = CbLoad<BM, 2 * WN_W>;

// ---------------------------------------------------------------------------
// Up/gate GEMM with SwiGLU epilogue. i = interleaved W_ug row, j = token slot
// (the weight is the A operand, so each lane's four consecutive i are four
// consecutive features of Z). Writes Z column-blocked [f/64][S][64] (S
// scratch slots in all); the state update reads the same blocks transposed,
// so Z is written once.
// grid: nx * ny workgroups, nx = 2f/256, ny = S/256
struct A1Args {
  const bf16_t *x;
  const bf16_t *Wug;
  bf16_t *Z;
  long long S;
  int d, f;
  int nx, ny;  // tiles along W_ug rows and along token slots
  Seqs sq;
};

__global__ __launch_bounds__(NT_W, 1) void k_a1(A1Args p) {
  __shared__ __attribute__((aligned(16))) Slab<WN_W, NBJ_W> ring[NSL_W];
  int tx, ty;  // W_ug tile, token tile
  band_tile(xcd_tile(blockIdx.x, gridDim.x), p.nx, p.ny, 8, tx, ty);
  const int n0 = tx * 256;
  const long long m0 = (long long)ty * BM;  // first slot of the tile
  const SeqInfo si = p.sq.at(p.sq.of_tile(ty));
  const int pos0 = (int)(m0 - si.slot0);
  SlabLoads<CbW, RmW> ld;
  ld.a.init(p.Wug + (long long)n0 * 64, 2LL * p.f * 64, 2 * p.f - n0, wave_id(), threadIdx.x & 63);
  ld.b.init(p.x + (si.xrow0 + pos0) * p.d, p.d, si.len - pos0, p.d, wave_id(), threadIdx.x & 63);
  Acc<NBJ_W> acc;
  acc_zero(acc);
  gemm_k<WN_W, NBJ_W, NSL_W, kARows>(acc, ring, ld, p.d / BK);

  // Epilogue. The wave's 128 W_ug rows are two (up, gate) pairs of 32-row
  // blocks: row fragments gi and gi + 2 (gi in 0, 1, 4, 5) hold matching up
  // and gate rows, features f0 + 32(gi/4) + 16(gi%2) + 4(l/16) + r with
  // f0 = n0/2 + 64 wm, a multiple of 64: all of the wave's features lie in
  // one 64-feature block of Z (f is a multiple of 256, so all are < f), and
  // its slots are s0 + 16gj + l%16, 64 consecutive ones. So the wave's part
  // of Z is one contiguous 8 KB run (64 slots x 128 bytes). It goes through
  // LDS (the ring, free once every wave is done with it): each lane writes
  // its 4 features of a slot (8 bytes), then reads back 16 bytes of a slot
  // row, and every store instruction writes 1 KB contiguous. Partial-line
  // stores (8-byte pieces, 32 contiguous bytes per slot row) measured 5%
  // slower on this kernel. The staging tile is [64 slots][64 features] with
  // the GEMM tiles' chunk swizzle (lds_off): the 16 rows one write
  // instruction touches at one column, and the 2 rows of 16 lanes of a read,
  // fall in distinct banks.
  static_assert(2 * WN_W * 64 * SK * 2 <= (int)sizeof(ring), "the staging tiles fit the ring");
  const int lane = threadIdx.x & 63, w = wave_id(), wm = w & 1, wn = w >> 1;
  const int f0 = n0 / 2 + wm * 64;
  const long long s0 = m0 + wn * 64;
  __syncthreads();  // every wave is done reading the ring
  bf16_t *stg = reinterpret_cast<bf16_t *>(ring) + w * 64 * SK;
#pragma unroll
  for (int gp = 0; gp < 4; ++gp) {
    const int gi = (gp >> 1) * 4 + (gp & 1);
#pragma unroll
    for (int gj = 0; gj < 2 * NBJ_W; ++gj) {
      const f32x4 &u = acc.v[gi][gj];
      const f32x4 &g = acc.v[gi + 2][gj];
      float z[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) z[r] = silu_fast(g[r]) * u[r];
      // features (gi/4)*32 + (gi%2)*16 + 4(l/16) .. +3: 16-byte chunk (gi/4)*4 + (gi%2)*2 + l/32, half (l/16)%2
      *reinterpret_cast<u32x2_t *>(stg + lds_off(16 * gj + (lane & 15), (gi >> 2) * 4 + (gi & 1) * 2 + (lane >> 5)) +
                                   4 * ((lane >> 4) & 1)) = u32x2_t{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
    }
  }
  // Z [f/64][S][64]: (slot, feature) at ((feature/64)*S + slot)*64 + feature%64; the wave's run starts at slot s0
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      p.Z + ((long long)(f0 / 64) * p.S + s0) * 64, (short)0, 0x7fffffff, kBufferFlags);
  constexpr int kNt = 2;  // cache policy of the stores: non-temporal
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // slot row 8k + l/8, bytes 16(l%8) .. +15 of it: byte 1024k + 16l of the run
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stg + lds_off(8 * k + (lane >> 3), lane & 7));
    __builtin_amdgcn_raw_buffer_store_b128(v, rz, (uint32_t)(lane * 16), k * 1024, kNt);
  }
}

// ---------------------------------------------------------------------------
// General target rows V = U W_target (U: tap sums of the token embeddings),
// written straight into the layouts the scan reads: V^T K-blocked
// [S/64][d][64] and, when clipping needs it, V row-major [S][d] (S scratch
// slots of all sequences). i = token slot, j = model dim a; the B operand is
// W_target^T [d][d] (row a holds column a of W_target). U rows past each
// sequence's length are zero, so are those of V.
// grid: nx * ny workgroups, nx = d/256, ny = S/256
struct TgtArgs {
  const bf16_t *U;
  const bf16_t *WtT;
  bf16_t *VT;    // eta * V
  bf16_t *Vrow;  // V
  float eta;
  int d, nx, ny;
  int round;  // workgroups resident at once (the compute units), a multiple of 8
};

__global__ __launch_bounds__(NT_W, 1) void k_target_gemm(TgtArgs p) {
  __shared__ __attribute__((aligned(16))) Slab<WN_W, NBJ_W> ring[NSL_W];
  int tx, ty;  // model-dim tile, token tile
  band_tile(xcd_tile_rounds(blockIdx.x, gridDim.x, p.round), p.nx, p.ny, 8, tx, ty);
  const int n0 = tx * 256;
  const long long m0 = (long long)ty * BM;  // first slot of the tile
  SlabLoads<RmW, RmW> ld;
  ld.a.init(p.U + (long long)m0 * p.d, p.d, BM, p.d, wave_id(), threadIdx.x & 63);
  ld.b.init(p.WtT + (long long)n0 * p.d, p.d, 256, p.d, wave_id(), threadIdx.x & 63);
  Acc<NBJ_W> acc;
  acc_zero(acc);
  gemm_k<WN_W, NBJ_W, NSL_W, kARows>(acc, ring, ld, p.d / BK);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
#pragma unroll
  for (int gj = 0; gj < 2 * NBJ_W; ++gj) {
    const int a = n0 + wn * WC_W + gj * 16 + (lane & 15);
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
        const long long pos = m0 + wm * 128 + gi * 16 + 4 * (lane >> 4);  // a slot
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc.v[gi][gj][r];
        uint2 pk;
        pk.x = pack_bf16x2(p.eta * v[0], p.eta * v[1]);
        pk.y = pack_bf16x2(p.eta * v[2], p.eta * v[3]);
        *reinterpret_cast<uint2 *>(p.VT + ((pos >> 6) * p.d + a) * 64 + (pos & 63)) = pk;
        if (p.Vrow) {
          bf16_t *vr = p.Vrow + pos * p.d + a;
#pragma unroll
          for (int r = 0; r < 4; ++r) vr[(long long)r * p.d] = f32_to_bf16(v[r]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// State update with snapshots. i = hidden unit (Z column), j = model dim (VT row),
// k = token slot. The state of a sequence is D = W - W0, the change of the
// fast weight since its last reset, in fp32; the accumulators of one tile
// hold it for the whole token stream. Because D starts at zero and stays
// small next to W, every rank-16 MFMA increment is added to a small number:
// increments far below the fp32 resolution of W itself (as with clipped
// updates) still accumulate with fp32 relative precision, also across calls.
// At each group start g*L the tile is written out as the bf16 snapshot
// bf16(W0 + D), with W0 read from the initial weight's bf16 planes.
//
// The state is cut into 256 x 256 tiles (i x a), numbered per sequence in
// bands of 8 along a (see band_tile) and then across sequences. Whole rounds
// of them (one per CU) run on the 8-wave configuration; a last partial round
// of at most 128 tiles is split into 256 x 128 halves that run as one round
// on the 4-wave configuration, so no CU idles for a whole round.

// Tile loads of the update with an L2 prefetch. Every Z tile (a band of
// 256 hidden units) is read by one XCD only, so its slabs come from HBM, one
// slab (two in the half-tile round) ahead of use without the prefetch. The
// workgroups that share an operand tile split its prefetch: the sa tiles (and
// halves) of a band of the tile order split the 256 lines of 128 bytes of a Z
// slab (4 blocks of 64 lines), the sb tiles along x of an XCD's range split
// the BN rows (one line each) of a V^T slab. Waves 0 .. WN-1 touch the first
// share, waves WN .. 2WN-1 the second, each with one 4-byte DMA into a
// 256-byte LDS sink that nothing reads; each lane's offset within the slab is
// fixed at the start. A wave's Z lines span at most two blocks (at most 64
// lines), so its offsets, from the first block it touches, stay below
// S*128 + 8 KB.
template <int WN, int BN>
struct UpdLoads : SlabLoads<ZbLoad<2 * WN>, KbLoad<BN, 2 * WN>> {
  static constexpr bool kPf = true;
  using Base = SlabLoads<ZbLoad<2 * WN>, KbLoad<BN, 2 * WN>>;
  // every load untracked (see dma16_untracked): the A tile is read transposed
  template <class S>
  __device__ __forceinline__ void issue(const typename Base::Pre &p, S &slab, int sl, int w, int lane, int j) const {
    if (j < ZbLoad<2 * WN>::N)
      this->a.issue(p.a, slab.a, sl, w, lane, j);
    else
      this->b.issue_untracked(p.b, slab.b, w, j - ZbLoad<2 * WN>::N);
  }
  uint32_t *sink;
  const bf16_t *pa;  // A sharers: the first Z block this wave touches, at the tile's first slot
  uint32_t vp;       // this lane's byte offset in the slab (A: from block pa, B: row)
  // sharer ka of sa takes lines [ka*256/sa, (ka+1)*256/sa) of the Z slab;
  // sharer kb of sb takes rows [kb*BN/sb, (kb+1)*BN/sb) of the V^T slab
  __device__ __forceinline__ void init_pf(uint32_t *sink_, const bf16_t *Z, long long S, int i0, long long slot0,
                                          int sa, int ka, int sb, int kb, int w, int lane) {
    sink = sink_;
    if (w < WN) {
      const int lo = ka * 256 / sa, n = (ka + 1) * 256 / sa - lo;
      const int per = (n + WN - 1) / WN < 64 ? (n + WN - 1) / WN : 64;
      const int first = lo + w * per < lo + n - 1 ? lo + w * per : lo + n - 1;
      int line = lo + w * per + lane % per;
      if (line > lo + n - 1) line = lo + n - 1;
      pa = Z + ((long long)(i0 / 64 + (first >> 6)) * S + slot0) * 64;
      vp = (uint32_t)(((line >> 6) - (first >> 6)) * S * 128 + (line & 63) * 128);
    } else {
      const int lo = kb * BN / sb, n = (kb + 1) * BN / sb - lo;
      const int per = (n + WN - 1) / WN < 64 ? (n + WN - 1) / WN : 64;
      int row = lo + (w - WN) * per + lane % per;
      if (row > lo + n - 1) row = lo + n - 1;
      vp = (uint32_t)(row * 128);
    }
  }
  __device__ __forceinline__ void prefetch(int sl, int w) const {
    const __amdgpu_buffer_rsrc_t rs =
        w < WN ? __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(pa + (long long)sl * 64 * 64), (short)0,
                                                   0x7fffffff, kBufferFlags)
               : __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(this->b.base + (long long)sl * this->b.kblk),
                                                   (short)0, 0x7fffffff, kBufferFlags);
    dma4_untracked(rs, sink, vp, 0);
  }
};

// LDS of the update: the ring and the prefetch sink (256 bytes that nothing reads).
template <int WN, int NBJ, int NSL>
struct UpdLds {
  Slab<WN, NBJ> ring[NSL];
  uint32_t sink[64];
};

struct UpdArgs {
  const bf16_t *Z;        // Z [f/64][S][64]
  const bf16_t *VT;
  const float *state_in;  // D [..][d][f], indexed by SeqInfo::state_in
  float *state_out;       // D [..][d][f], indexed by SeqInfo::state_out
  bf16_t *snap;
  const bf16_t *W0p;      // W0 as planes [f/8][d][8]
  long long S;            // scratch slots in all (Z's block stride is S*64)
  int L, d, f;
  int tile0;  // first 256 x 256 tile of this launch
  int round;  // workgroups resident at once (the compute units), a multiple of 8
  Seqs sq;
};

// Snapshots W[a][i] are held as planes of 8 columns ([f/8][d][8]: element
// (a, i) at ((i/8)*d + a)*8 + i%8). The MFMA accumulator layout gives lane l
// four consecutive i of one a per accumulator: i = 4*(l/16) .. +3 of the
// tile's 16, a = l%16. Snapshots are written, and the initial weight read
// back, 16 bytes per lane in an exchanged layout: for the accumulators
// (gi, 2gp) and (gi, 2gp+1), 16 a apart, lanes 0-15 hold the eight i 0-7 (one
// 16-byte chunk of a plane) of the first, lanes 16-31 those of the second,
// and lanes 32-63 the same for i 8-15, the next plane. One instruction then
// covers 32 consecutive a of two planes: two runs of 512 contiguous bytes.
// v_permlane16_swap trades the odd 16-lane rows of its first operand for the
// even rows of its second; applied to the low and high halves of each lane's
// chunk it turns the exchanged layout into the two accumulators' layout, and
// back (it is its own inverse).
// A lane offset locates this lane's chunk for (gi, gp) = (0, 0):
// a = j0 + wn*32*NBJ + l%32, plane (i0 + wm*128)/8 + l/32; tiles are always
// full (d, f multiples of 256). Pair (gi, gp) lies 2gi planes and 32gp rows
// of a further on.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Swaps the odd 16-lane rows of a with the even rows of b.
__device__ __forceinline__ void swap_rows16(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// A VALU write to the data registers of a buffer store wider than 8 bytes
// must come at least two wait states after the store, or the store may write
// the new values. The compiler counts them for such stores with a constant
// soffset but not with a register soffset (the snapshot stores take their
// plane offset there), so they are explicit here.
__device__ __forceinline__ void guard_wide_store() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);
}

// The initial weight W0 as bf16 planes ([f/8][d][8], the snapshot layout): a
// buffer descriptor over them and this lane's byte offset in the exchanged
// layout, so that each load is one instruction with a scalar offset (64-bit
// addresses per load would cost two registers each).
struct QRead {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vo;
  int d;
  // byte offsets of pair (gi, gp): 2gi planes of 8 columns in the scalar
  // offset, 32gp rows (gp*256 elements) in the lane offset (an immediate)
  __device__ __forceinline__ int soff(int gi) const { return gi * 32 * d; }
  __device__ __forceinline__ u32x4_t load(int gi, int gp) const {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, vo + gp * 512, soff(gi), 0);
  }
};

// Snapshot of the weight W0 + D: bf16(W0 + D) into the snapshot planes at
// `snap` (one group's [f/8][d][8] planes), with the accumulators holding D
// (read, not changed) and W0 read back from the initial weight's bf16 planes,
// with the same lane and scalar offsets (the two share their layout). All
// loads go out before the first add (one memory round trip); the scheduling
// barriers keep the compiler from moving them. The snapshot runs between
// stages, when the MFMA fragments are dead, so their 64 registers fit. The
// stores are non-temporal: no kernel of the update reads them, and they would
// evict operand slabs that other workgroups still read from L2.
template <int NBJ>
__device__ __forceinline__ void dump_snapshot(const Acc<NBJ> &acc, const QRead &qr, const bf16_t *snap) {
  constexpr int kNt = 2;
  constexpr int NTOT = 8 * NBJ;  // 8 row fragments x NBJ pairs of column fragments
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(snap), (short)0, 0x7fffffff, kBufferFlags);
  u32x4_t qv[NTOT];
  pin();
#pragma unroll
  for (int k = 0; k < NTOT; ++k) qv[k] = qr.load(k & 7, k >> 3);
#pragma unroll
  for (int k = 0; k < NTOT; ++k) {
    const int gi = k & 7, gp = k >> 3;
    const f32x4 &u = acc.v[gi][2 * gp];
    const f32x4 &v = acc.v[gi][2 * gp + 1];
    // W0 in the accumulators' layout: after the two swaps w0, w1 hold this
    // lane's four i of accumulator (gi, 2gp) and w2, w3 those of (gi, 2gp+1)
    uint32_t w0 = qv[k].x, w1 = qv[k].y, w2 = qv[k].z, w3 = qv[k].w;
    swap_rows16(w0, w2);
    swap_rows16(w1, w3);
    uint32_t p0 = pack_bf16x2(u[0] + bf16_lo(w0), u[1] + bf16_hi(w0));
    uint32_t p1 = pack_bf16x2(u[2] + bf16_lo(w1), u[3] + bf16_hi(w1));
    uint32_t p2 = pack_bf16x2(v[0] + bf16_lo(w2), v[1] + bf16_hi(w2));
    uint32_t p3 = pack_bf16x2(v[2] + bf16_lo(w3), v[3] + bf16_hi(w3));
    // and back to the exchanged layout: eight consecutive i of one a per lane
    swap_rows16(p0, p2);
    swap_rows16(p1, p3);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{p0, p1, p2, p3}, rs, qr.vo + gp * 512, qr.soff(gi), kNt);
    guard_wide_store();
  }
  pin();
}

// WN = 4: workgroup n of the launch is tile tile0 + n (a 256 x 256 tile);
// WN = 2: workgroup n is half n%2 (128 columns of a) of tile tile0 + n/2.
template <int WN, int NBJ, int NSL>
__global__ __launch_bounds__(128 * WN, 1) void k_update(UpdArgs p) {
  __shared__ __attribute__((aligned(16))) UpdLds<WN, NBJ, NSL> lds;
  Slab<WN, NBJ> *ring = lds.ring;
  constexpr int BN = 32 * WN * NBJ;  // columns of a per workgroup
  const int nx = p.f / BM, ny = p.d / 256;
  const int n = xcd_tile_rounds(blockIdx.x, gridDim.x, p.round);
  const int t = p.tile0 + n / (256 / BN);
  const int b = t / (nx * ny);  // sequence
  const SeqInfo si = p.sq.at(b);
  int tx, ty;
  band_tile(t - b * nx * ny, nx, ny, 8, tx, ty);
  const int i0 = tx * BM;
  const int j0 = ty * 256 + (n % (256 / BN)) * BN;
  const int lane = threadIdx.x & 63;
  const int w = wave_id(), wm = w & 1, wn = w >> 1;
  const long long df = (long long)p.d * p.f;
  // this lane's first element of the tile in the state ([d][f]), and its first 16-byte chunk of a
  // snapshot ([f/8][d][8]) in the exchanged layout of the snapshot accesses
  const long long lane_off =
      (long long)(j0 + wn * 32 * NBJ + (lane & 15)) * p.f + i0 + wm * 128 + 4 * (lane >> 4);
  const long long lane_snap =
      (long long)((i0 + wm * 128) / 8 + (lane >> 5)) * 8 * p.d + (j0 + wn * 32 * NBJ + (lane & 31)) * 8;
  const bf16_t *snap0 = p.snap + (long long)si.grp0 * df;
  const int ngroups = si.len > p.L ? (si.len + p.L - 1) / p.L : 1;
  // where this lane's part of the final state goes (null: nowhere)
  float *st_out = si.state_out >= 0 ? p.state_out + si.state_out * df + lane_off : nullptr;

  Acc<NBJ> acc;
  if (si.state_in >= 0) {
    const float *st = p.state_in + si.state_in * df + lane_off;
#pragma unroll
    for (int gj = 0; gj < 2 * NBJ; ++gj) {
      const float *row = st + (long long)gj * 16 * p.f;
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const float4 v = *reinterpret_cast<const float4 *>(row + gi * 16);
        acc.v[gi][gj][0] = v.x;
        acc.v[gi][gj][1] = v.y;
        acc.v[gi][gj][2] = v.z;
        acc.v[gi][gj][3] = v.w;
      }
    }
  } else {
    acc_zero(acc);  // a document start: W = W0
  }

  // A: Z blocks [f/64][S][64], read transposed; B: eta V^T K-blocked [S/64][d][64]
  UpdLoads<WN, BN> ld;
  ld.a.init(p.Z, p.S, i0, si.slot0, w, lane);
  ld.b.init(p.VT + (long long)si.slot0 * p.d + (long long)j0 * 64, (long long)p.d * 64, w, lane);
  {
    // Z tile tx is shared by the tiles of its band (h of them) and their halves;
    // a V^T tile (or half) by the tiles along x of the XCD's range
    const int full = ny / 8, band = ty / 8, h = band < full ? 8 : ny - full * 8;
    const int halves = 256 / BN, half = n % halves;
    ld.init_pf(lds.sink, p.Z, p.S, i0, si.slot0, h * halves, (ty - band * 8) * halves + half, 16 / WN, tx % (16 / WN),
               w, lane);
  }
  const int nk = (si.len + BK - 1) / BK;
  QRead qr;
  qr.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(p.W0p), (short)0, (int)(df * 2), kBufferFlags);
  qr.vo = (uint32_t)(lane_snap * 2);
  qr.d = p.d;
  // Snapshot 0 is the entry weight. Group starts are multiples of the stage
  // depth, so snapshot g is written right after the last stage of group g-1,
  // while the following slabs are already in flight.
  dump_snapshot(acc, qr, snap0);
  int g = 1;
  const int nsl = (nk + 1) >> 1;
  Frag<NBJ> fr;
  if (nk > 0) {
    ring_prologue<WN, NBJ, NSL>(ld, [&](int sl) -> Slab<WN, NBJ> & { return ring[sl]; }, nsl, w, lane);
    read_a<WN, NBJ, kAZ>(fr.lo, ring[0], 0, 0, wm, lane);
    read_b<WN, NBJ>(fr.b[0], ring[0], 0, wn, lane);
  }
  // The snapshot stores share the vector-memory counter with the tile loads.
  // The counted waits stay exact for the loads: loads complete in issue
  // order among themselves, so while a load is outstanding every later load
  // is too, and the count exceeds the number allowed; a store in flight can
  // only make a wait last longer.
  auto snapshot = [&](const Acc<NBJ> &a) {
    dump_snapshot(a, qr, snap0 + (long long)g * df);
    ++g;
  };
  // Stages of group g-1 run plain; its last stage ends with snapshot g.
  // A group spans L/BK stages, an even number (L is a multiple of 64), so
  // every group ends on an odd stage.
  int kt = 0, cb = 0;  // cb: the ring buffer of slab kt/2
  while (g < ngroups) {  // the snapshot advances g
    const int kt_last = g * (p.L / BK) - 1;  // last stage before group g starts
    stage_run<WN, NBJ, NSL, kAZ>(acc, ring, fr, kt, cb, kt_last, nk, wm, wn, lane, w, ld);
    const int nb = cb + 1 == NSL ? 0 : cb + 1;
    stage_body<WN, NBJ, NSL, true, kAZ, 1, -1>(acc, ring[cb], ring[nb], fr, kt, nk, wm, wn, lane, w, ld, snapshot);
    cb = nb;
    ++kt;
  }
  stage_run<WN, NBJ, NSL, kAZ>(acc, ring, fr, kt, cb, nk, nk, wm, wn, lane, w, ld);
  // the final state D in fp32
  if (!st_out) return;
#pragma unroll
  for (int gj = 0; gj < 2 * NBJ; ++gj) {
    float *row = st_out + (long long)gj * 16 * p.f;
#pragma unroll
    for (int gi = 0; gi < 8; ++gi)
      *reinterpret_cast<float4 *>(row + gi * 16) =
          make_float4(acc.v[gi][gj][0], acc.v[gi][gj][1], acc.v[gi][gj][2], acc.v[gi][gj][3]);
  }
}

// ---------------------------------------------------------------------------
// Within-group scores P[t][s] = <z_t, z_s> for s in an earlier chunk of the
// same group. i = s, j = t; only tiles with i-tile <= j-tile that hold an
// unmasked entry are formed.
// grid: B * ngroups * nt(nt+1)/2 workgroups, nt = ceil(L/256)
constexpr int kMaxScorePairs = 136;  // the lower triangle of 16 x 16 tiles (L <= 4096)
// A pair entry (kPackedPair, a): with C = 128 the diagonal tiles a and a+1
// of a group, each holding two chunks, share one workgroup (below).
constexpr unsigned char kPackedPair = 0xff;

struct ScoreArgs {
  const bf16_t *Z;
  bf16_t *P;
  long long S;  // scratch slots in all (Z's block stride is S*64)
  int L, C, f, nt;
  int round;  // workgroups resident at once (the compute units), a multiple of 8
  Seqs sq;
  // tiles (it, jt) of a full group that hold an unmasked entry, and packed
  // diagonal pairs (kPackedPair, a); npairs = 0: every tile of the lower
  // triangle gets a workgroup (long groups)
  int npairs;
  unsigned char pit[kMaxScorePairs], pjt[kMaxScorePairs];
};

__global__ __launch_bounds__(NT_W, 1) void k_scores(ScoreArgs p) {
  __shared__ __attribute__((aligned(16))) Slab<WN_W, NBJ_W> ring[NSL_W];
  const int t = xcd_tile_rounds(blockIdx.x, gridDim.x, p.round);
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
  // bg: the group across all sequences
  const SeqInfo si = p.sq.at(p.sq.of_group(bg));
  const int gs = (bg - si.grp0) * p.L;       // first token of the group in its sequence
  const int Lg = si.len - gs < p.L ? si.len - gs : p.L;
  const int tp = (si.len + 255) & ~255;      // the sequence's slots
  // A packed pair (C = 128): of diagonal tile k (tokens 256k .. 256k+255,
  // chunks 2k and 2k+1) only s in chunk 2k against t in chunk 2k+1 is
  // unmasked, and the output GEMM also reads the all-masked block of t and s
  // in chunk 2k (as zeros). One workgroup takes tiles a and b = a+1: its rows
  // are s in chunk 2a, then chunk 2b; its columns t in chunk 2a+1, then
  // chunk 2b+1. The two diagonal quadrants are the unmasked blocks; the two
  // cross quadrants write the zero blocks of a and b.
  const bool packed = it == kPackedPair;
  const int i0 = packed ? jt * 256 : it * BM, j0 = packed ? jt * 256 + 128 : jt * 256;
  if (packed ? i0 >= Lg : j0 >= Lg) return;
  // A tile whose every s lies in the chunk of its last t or later is all
  // masked; the output GEMM never reads it (it stops before that chunk).
  const int jl = (j0 + 255 < Lg - 1) ? j0 + 255 : Lg - 1;
  if (!packed && i0 / p.C >= jl / p.C) return;
  const bf16_t *Zg = p.Z + ((long long)si.slot0 + gs) * 64;  // Z column-blocked [f/64][S][64]
  const long long zblk = p.S * 64;
  SlabLoads<CbW, CbW> ld;
  const int gap = packed ? 128 : 0;
  ld.a.init(Zg + (long long)i0 * 64, zblk, tp - gs - i0, wave_id(), threadIdx.x & 63, gap);
  ld.b.init(Zg + (long long)j0 * 64, zblk, tp - gs - j0, wave_id(), threadIdx.x & 63, gap);
  Acc<NBJ_W> acc;
  acc_zero(acc);
  gemm_k<WN_W, NBJ_W, NSL_W, kARows>(acc, ring, ld, p.f / BK);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  bf16_t *Pg = p.P + (long long)bg * p.L * p.L;
  if (packed) {
    // wave rows are s of tile k = a + wm; columns of the same half are t of
    // chunk 2k+1 (computed), of the other half t of chunk 2k (zeros)
    const int k = jt + wm;
#pragma unroll
    for (int gj = 0; gj < 2 * NBJ_W; ++gj) {
      const int c = wn * WC_W + gj * 16 + (lane & 15);
      const bool diag = (c >> 7) == wm;
      const int t = 256 * k + (diag ? 128 : 0) + (c & 127);
      if (t >= p.L) continue;
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const int sidx = 256 * k + gi * 16 + 4 * (lane >> 4);
        uint2 pk;
        pk.x = diag ? pack_bf16x2(acc.v[gi][gj][0], acc.v[gi][gj][1]) : 0u;
        pk.y = diag ? pack_bf16x2(acc.v[gi][gj][2], acc.v[gi][gj][3]) : 0u;
        *reinterpret_cast<uint2 *>(Pg + (long long)t * p.L + sidx) = pk;
      }
    }
    return;
  }
#pragma unroll
  for (int gj = 0; gj < 2 * NBJ_W; ++gj) {
    const int t = j0 + wn * WC_W + gj * 16 + (lane & 15);
    if (t >= p.L) continue;
    const int ct = t / p.C;
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
        const int sidx = i0 + wm * 128 + gi * 16 + 4 * (lane >> 4);
        if (sidx >= p.L) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = ((sidx + r) / p.C < ct) ? acc.v[gi][gj][r] : 0.f;
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(Pg + (long long)t * p.L + sidx) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// Snapshot with no update: snap[((i/8)*d + a)*8 + i%8] = bf16(W0[a][i] + D[a][i])
// (fp32 W0 and state D, [d][f] each). Thread (plane, a) converts one
// 8-column chunk.
__global__ __launch_bounds__(256) void k_state_to_snap(const float *W0, const float *D, bf16_t *snap, int d, int f) {
  const long long n = (long long)d * (f / 8);
  for (long long t = blockIdx.x * 256LL + threadIdx.x; t < n; t += (long long)gridDim.x * 256) {
    const int a = (int)(t % d);
    const long long pl = t / d;
    const long long o = (long long)a * f + pl * 8;
    const float4 w0 = *reinterpret_cast<const float4 *>(W0 + o), w1 = *reinterpret_cast<const float4 *>(W0 + o + 4);
    const float4 d0 = *reinterpret_cast<const float4 *>(D + o), d1 = *reinterpret_cast<const float4 *>(D + o + 4);
    uint4 pk;
    pk.x = pack_bf16x2(w0.x + d0.x, w0.y + d0.y);
    pk.y = pack_bf16x2(w0.z + d0.z, w0.w + d0.w);
    pk.z = pack_bf16x2(w1.x + d1.x, w1.y + d1.y);
    pk.w = pack_bf16x2(w1.z + d1.z, w1.w + d1.w);
    *reinterpret_cast<uint4 *>(snap + t * 8) = pk;
  }
}

// The initial weight as planes: dst[((i/8)*d + a)*8 + i%8] = src[a][i] (bf16, [d][f]).
__global__ __launch_bounds__(256) void k_to_planes(const bf16_t *src, bf16_t *dst, int d, int f) {
  const long long n = (long long)d * (f / 8);
  for (long long t = blockIdx.x * 256LL + threadIdx.x; t < n; t += (long long)gridDim.x * 256) {
    const int a = (int)(t % d);
    const long long pl = t / d;
    *reinterpret_cast<uint4 *>(dst + t * 8) = *reinterpret_cast<const uint4 *>(src + (long long)a * f + pl * 8);
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
  void *y;    // bf16 rows of d, or fp32 with y_f32
  long long S;  // scratch slots in all
  int L, C, d, f, intra;
  int y_f32;
  int round;  // workgroups resident at once (the compute units), a multiple of 8
  Seqs sq;
};

constexpr int LY_F = 260;  // [128 tokens][256 model dims + pad]: one half of an fp32 y tile
static_assert(128 * LY_F * 4 <= kSmemOut, "the fp32 y half tile fits the output GEMM's LDS");

__global__ __launch_bounds__(NT_W, 1) void k_out(OutArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[kSmemOut / 2];
  Slab<WN_W, NBJ_W> *ring = reinterpret_cast<Slab<WN_W, NBJ_W> *>(smem);
  // one group's tiles are consecutive, token tiles fastest; the chip takes
  // them in rounds, each XCD a contiguous range of a round
  const int nx = p.d / BM, ny = (p.L + 255) / 256;
  const int t = xcd_tile_rounds(blockIdx.x, gridDim.x, p.round);
  const int bg = t / (nx * ny), r = t - bg * nx * ny;  // bg: the group across all sequences
  const int i0 = (r / ny) * BM;
  const int j0 = (r % ny) * 256;
  const SeqInfo si = p.sq.at(p.sq.of_group(bg));
  const int gs = (bg - si.grp0) * p.L;  // first token of the group in its sequence
  const int Lg = si.len - gs < p.L ? si.len - gs : p.L;
  const int tp = (si.len + 255) & ~255;
  if (j0 >= Lg) return;
  const int w8 = wave_id(), l8 = threadIdx.x & 63;
  Acc<NBJ_W> acc;
  acc_zero(acc);
  {  // segment 1: the group's snapshot ([f/8][d][8] planes) against Z, K = f
    SlabLoads<PlLoad<2 * WN_W>, CbW> ld;
    ld.a.init(p.snap + (long long)bg * p.d * p.f + (long long)i0 * 8, (long long)p.d * 8, l8);
    ld.b.init(p.Z + ((long long)si.slot0 + gs + j0) * 64, p.S * 64, tp - gs - j0, w8, l8);
    gemm_k<WN_W, NBJ_W, NSL_W, kAPlanes>(acc, ring, ld, p.f / BK);
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
      ld.a.init(p.VT + ((long long)si.slot0 + gs) * p.d + (long long)i0 * 64, (long long)p.d * 64, w8, l8);
      ld.b.init(p.P + (long long)bg * p.L * p.L + (long long)j0 * p.L, p.L, p.L - j0, kv, w8, l8);
      __syncthreads();  // every wave is done reading the ring before it is refilled
      gemm_k<WN_W, NBJ_W, NSL_W, kARows>(acc, ring, ld, nk2);
    }
  }

  // Epilogue through LDS ([token][model dim]) so y rows leave in whole lines.
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), wm = w & 1, wn = w >> 1;
  if (p.y_f32) {
    // fp32 y: two halves of 128 tokens (waves 0-3 hold tokens 0-127, waves 4-7 the rest), 1 KB rows
    float *lf = reinterpret_cast<float *>(smem);
    float *yb = static_cast<float *>(p.y) + (si.xrow0 + gs + j0) * p.d + i0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      __syncthreads();  // the ring, or the first half's rows, are no longer read
      if ((wn >> 1) == half) {
#pragma unroll
        for (int gj = 0; gj < 2 * NBJ_W; ++gj) {
          const int tl = (wn & 1) * WC_W + gj * 16 + (lane & 15);
#pragma unroll
          for (int gi = 0; gi < 8; ++gi) {
            const int al = wm * 128 + gi * 16 + 4 * (lane >> 4);
            *reinterpret_cast<float4 *>(lf + tl * LY_F + al) =
                make_float4(acc.v[gi][gj][0], acc.v[gi][gj][1], acc.v[gi][gj][2], acc.v[gi][gj][3]);
          }
        }
      }
      __syncthreads();
      // 128 token rows x 1 KB; rows past the group's end are not written
#pragma unroll
      for (int it = 0; it < 8192 / NT_W; ++it) {
        const int idx = it * NT_W + tid;
        const int tr = idx >> 6, ch = idx & 63;
        if (j0 + half * 128 + tr < Lg)
          *reinterpret_cast<float4 *>(yb + (long long)(half * 128 + tr) * p.d + ch * 4) =
              *reinterpret_cast<const float4 *>(lf + tr * LY_F + ch * 4);
      }
    }
    return;
  }
  bf16_t *ly = smem;
  __syncthreads();  // every wave is done with the ring
#pragma unroll
  for (int gj = 0; gj < 2 * NBJ_W; ++gj) {
    const int tl = wn * WC_W + gj * 16 + (lane & 15);
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
      const int al = wm * 128 + gi * 16 + 4 * (lane >> 4);
      uint2 pk;
      pk.x = pack_bf16x2(acc.v[gi][gj][0], acc.v[gi][gj][1]);
      pk.y = pack_bf16x2(acc.v[gi][gj][2], acc.v[gi][gj][3]);
      *reinterpret_cast<uint2 *>(ly + tl * LY_P + al) = pk;
    }
  }
  __syncthreads();
  // 256 token rows x 512 bytes; rows past the group's end are not written
  bf16_t *yb = static_cast<bf16_t *>(p.y);
#pragma unroll
  for (int it = 0; it < 8192 / NT_W; ++it) {
    const int idx = it * NT_W + tid;
    const int tr = idx >> 5, ch = idx & 31;
    if (j0 + tr < Lg)
      *reinterpret_cast<uint4 *>(yb + (si.xrow0 + gs + j0 + tr) * p.d + i0 + ch * 8) =
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
  const bf16_t *Z;     // column-blocked [f/64][S][64]
  const bf16_t *V;     // [S][d], rows past each sequence's length zero (without GATHER)
  const bf16_t *E;     // [vocab][d] (GATHER)
  const int32_t *ids;  // the caller's ids, a sequence's at SeqInfo::id0 (GATHER)
  float *gv;           // scratch: 256 KB per workgroup of the grid
  float *rowpart;      // [S/256][wspan][256]
  int C, d, f, wspan, vocab;
  long long S;         // scratch slots in all: Z's block stride is S*64
  int round;           // workgroups resident at once (the compute units), a multiple of 8
  Seqs sq;
};

constexpr int GR_P = 129;  // fp32 pitch of a [256][128] product tile in LDS (conflict-free row sums)
constexpr int kSmemGram = cmax(kRingBytes, 256 * GR_P * 4);

template <bool GATHER>
__global__ __launch_bounds__(NT_W, 1) void k_chunk_gram(GramArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemGram];
  Slab<WN_W, NBJ_W> *ring = reinterpret_cast<Slab<WN_W, NBJ_W> *>(smem);
  const int id = xcd_tile_rounds(blockIdx.x, gridDim.x, p.round);  // the t-tiles of an s-tile share an XCD
  const int wr = id % p.wspan;
  const int u = id / p.wspan;  // the s-tile: 256 slots of one sequence
  const SeqInfo si = p.sq.at(p.sq.of_tile(u));
  const int len = si.len, tp = (len + 255) & ~255;  // positions and slots of the sequence
  const int s0 = (int)((long long)u * 256 - si.slot0);  // position of the s-tile in its sequence
  float *out = p.rowpart + ((long long)u * p.wspan + wr) * 256;
  const int s_last = (s0 + 255 < len - 1) ? s0 + 255 : len - 1;
  const int w = (int)((long long)(s0 / p.C) * p.C / 256) + wr;
  const long long w_end = (((long long)(s_last / p.C) + 1) * p.C - 1) / 256;
  const int w_hi = (int)(w_end < tp / 256 - 1 ? w_end : tp / 256 - 1);
  if (s0 >= len || w > w_hi) {  // no token pair of this tile shares a chunk
    if (threadIdx.x < 256) out[threadIdx.x] = 0.f;
    return;
  }
  const int t0 = w * 256;
  const int lane = threadIdx.x & 63, wv = wave_id(), wm = wv & 1, wn = wv >> 1;
  Acc<NBJ_W> acc;
  acc_zero(acc);
  if constexpr (GATHER) {
    SlabLoads<RmGather<BM, 2 * WN_W>, RmGather<BM, 2 * WN_W>> ld;
    const int32_t *tg = p.ids + si.id0 + 1;  // target id of position q at tg[q]
    ld.a.init(p.E, p.d, p.vocab, tg + s0, len - s0, wv, lane);
    ld.b.init(p.E, p.d, p.vocab, tg + t0, len - t0, wv, lane);
    gemm_k<WN_W, NBJ_W, NSL_W, kARows>(acc, ring, ld, p.d / BK);
  } else {
    const bf16_t *Vb = p.V + (long long)si.slot0 * p.d;
    SlabLoads<RmW, RmW> ld;
    ld.a.init(Vb + (long long)s0 * p.d, p.d, tp - s0, p.d, wv, lane);
    ld.b.init(Vb + (long long)t0 * p.d, p.d, tp - t0, p.d, wv, lane);
    gemm_k<WN_W, NBJ_W, NSL_W, kARows>(acc, ring, ld, p.d / BK);
  }
  // G_V to this lane's scratch: accumulator k = gi*2*NBJ + gj (4 registers) at [k][lane]
  float4 *gv = reinterpret_cast<float4 *>(p.gv) + ((long long)id * 8 + wv) * (32 * 64) + lane;
#pragma unroll
  for (int gi = 0; gi < 8; ++gi)
#pragma unroll
    for (int gj = 0; gj < 2 * NBJ_W; ++gj)
      gv[(gi * 2 * NBJ_W + gj) * 64] =
          make_float4(acc.v[gi][gj][0], acc.v[gi][gj][1], acc.v[gi][gj][2], acc.v[gi][gj][3]);
  __syncthreads();  // the second pass refills the ring
  acc_zero(acc);
  {
    const bf16_t *Zb = p.Z + (long long)si.slot0 * 64;  // Z column-blocked [f/64][S][64]
    SlabLoads<CbW, CbW> ld;
    ld.a.init(Zb + (long long)s0 * 64, p.S * 64, tp - s0, wv, lane);
    ld.b.init(Zb + (long long)t0 * 64, p.S * 64, tp - t0, wv, lane);
    gemm_k<WN_W, NBJ_W, NSL_W, kARows>(acc, ring, ld, p.f / BK);
  }
  // products of same-chunk pairs, in place of G_Z: row s0 + sl shares column
  // t's chunk when lo <= sl < lo + C (lo: the chunk's start less s0); four
  // accumulators at a time, so few reloaded values are live at once
#pragma unroll
  for (int gj = 0; gj < 2 * NBJ_W; ++gj) {
    const int lo = (t0 + wn * WC_W + gj * 16 + (lane & 15)) / p.C * p.C - s0;
#pragma unroll
    for (int g4 = 0; g4 < 8; g4 += 4) {
      pin();
#pragma unroll
      for (int gi = g4; gi < g4 + 4; ++gi) {
        const float4 g = gv[(gi * 2 * NBJ_W + gj) * 64];
        const float gq[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sl = wm * 128 + gi * 16 + 4 * (lane >> 4) + r;
          const float e = acc.v[gi][gj][r];
          acc.v[gi][gj][r] = (sl >= lo && sl < lo + p.C) ? e * gq[r] : 0.f;
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
      for (int gj = 0; gj < 2 * NBJ_W; ++gj) {
        const int tl = (wn & 1) * WC_W + gj * 16 + (lane & 15);
#pragma unroll
        for (int gi = 0; gi < 8; ++gi)
#pragma unroll
          for (int r = 0; r < 4; ++r) tile[(wm * 128 + gi * 16 + 4 * (lane >> 4) + r) * GR_P + tl] = acc.v[gi][gj][r];
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
// Target gather, transposed and K-blocked: V^T[p/64][a][p%64] = eta * E[ids of slot p's next token][a]
// (slots across all sequences). A 64-slot x 64-feature tile passes through LDS so both the row reads of E and
// the writes (one contiguous 8 KB block) are 16 B per lane. With Vrow non-null
// the rows are also written row-major, Vrow[p][a] (used by update clipping).
// With cfac non-null, position t of sequence b is also scaled by the clipping factor cfac[b][t/C]
// (bf16 -> fp32, times eta and the factor, rounded to bf16). Vrow holds the unscaled rows.
// grid: (S/64, d/64)
__global__ __launch_bounds__(256) void k_gather_vt(const int32_t *ids, const bf16_t *E, int vocab, bf16_t *VT,
                                                   bf16_t *Vrow, const float *cfac, float eta, int C, int nchunks,
                                                   int d, Seqs sq) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64][72];
  const long long p0 = (long long)blockIdx.x * 64;
  const int a0 = blockIdx.y * 64;
  const int b = sq.of_tile((int)(p0 / 256));
  const SeqInfo si = sq.at(b);
  const int q0 = (int)(p0 - si.slot0);  // position of the block's first slot in its sequence
  const int tid = threadIdx.x, seg = tid & 7;
  // both passes' ids, then both rows: the loads overlap instead of waiting in turn
  int id[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int pos = q0 + pass * 32 + (tid >> 3);
    id[pass] = pos < si.len ? ids[si.id0 + pos + 1] : -1;
  }
  // unconditional loads (an id outside [0, vocab) reads row 0, then zero): a
  // load behind a branch would wait for itself before the next one
  uint4 row[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const bool ok = id[pass] >= 0 && id[pass] < vocab;
    const uint4 r = *reinterpret_cast<const uint4 *>(E + (long long)(ok ? id[pass] : 0) * d + a0 + seg * 8);
    row[pass] = ok ? r : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int pl = pass * 32 + (tid >> 3);
    const int pos = q0 + pl;
    const uint4 v = row[pass];
    if (Vrow) *reinterpret_cast<uint4 *>(Vrow + (p0 + pl) * d + a0 + seg * 8) = v;  // unscaled
    // V^T carries eta (and the clipping factor): bf16 -> fp32, scaled, rounded to bf16
    const float c = eta * ((cfac && pos < si.len) ? cfac[(long long)b * nchunks + pos / C] : 1.f);
    uint4 sv;
    {
      const bf16_t *e = reinterpret_cast<const bf16_t *>(&v);
      uint32_t *o = reinterpret_cast<uint32_t *>(&sv);
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(bf16_to_f32(e[2 * k]) * c, bf16_to_f32(e[2 * k + 1]) * c);
    }
    // 16-byte column groups XOR-swizzled by (row / 8) % 8: the transposing
    // reads below take one column from rows 8 apart, which the plain layout
    // puts in the same banks
    *reinterpret_cast<uint4 *>(&tile[pl][(seg ^ ((pl >> 3) & 7)) * 8]) = sv;
  }
  __syncthreads();
  bf16_t *blk = VT + (long long)blockIdx.x * d * 64;
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
                                 const float *cfac, float eta, const Layout &lay, hipStream_t s) {
  if (lay.n_slots() / 64 >= (1LL << 31)) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)(lay.n_slots() / 64), lay.d / 64, 1);
  const int nchunks = (int)((lay.T + (long long)lay.C - 1) / lay.C);
  hipLaunchKernelGGL(k_gather_vt, grid, dim3(256), 0, s, ids, E, vocab, VT, Vrow, cfac, eta, lay.C, nchunks, lay.d,
                     lay.seqs());
  return hipGetLastError();
}

hipError_t launch_chunk_gram_bf16(const bf16_t *Z, const bf16_t *Vrow, const bf16_t *E, const int32_t *ids, int vocab,
                                  float *gv, float *rowpart, int wspan, const Layout &lay, int cus, hipStream_t s) {
  const long long n = lay.n_slots() / 256 * wspan;
  if (n >= (1LL << 31) / 8) return hipErrorInvalidConfiguration;
  if (!Vrow && (long long)vocab * lay.d * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  GramArgs p{Z, Vrow, E, ids, gv, rowpart, lay.C, lay.d, lay.f, wspan, vocab, lay.n_slots(), launch_round(cus),
             lay.seqs()};
  if (Vrow)
    hipLaunchKernelGGL(k_chunk_gram<false>, dim3((unsigned)n), dim3(NT_W), 0, s, p);
  else
    hipLaunchKernelGGL(k_chunk_gram<true>, dim3((unsigned)n), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_a1_bf16(const bf16_t *x, const bf16_t *Wug, bf16_t *Z, const Layout &lay, hipStream_t s) {
  const int nx = (2 * lay.f + 255) / 256;
  const long long ny = lay.n_slots() / BM;
  if (nx * ny >= (1LL << 31)) return hipErrorInvalidConfiguration;
  A1Args p{x, Wug, Z, lay.n_slots(), lay.d, lay.f, nx, (int)ny, lay.seqs()};
  hipLaunchKernelGGL(k_a1, dim3((unsigned)(nx * ny)), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_target_gemm_bf16(const bf16_t *U, const bf16_t *WtT, bf16_t *VT, bf16_t *Vrow, float eta,
                                  const Layout &lay, int cus, hipStream_t s) {
  const int nx = lay.d / 256;
  const long long ny = lay.n_slots() / BM;
  if (nx * ny >= (1LL << 31)) return hipErrorInvalidConfiguration;
  TgtArgs p{U, WtT, VT, Vrow, eta, lay.d, nx, (int)ny, launch_round(cus)};
  hipLaunchKernelGGL(k_target_gemm, dim3((unsigned)(nx * ny)), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_update_bf16(const bf16_t *Z, const bf16_t *VT, const float *state_in, float *state_out,
                              bf16_t *snap, const bf16_t *W0p, const Layout &lay, int cus, hipStream_t s) {
  const long long tiles = (long long)lay.n_seq() * (lay.f / BM) * (lay.d / 256);
  if (tiles * 2 >= (1LL << 31)) return hipErrorInvalidConfiguration;
  // the Z prefetch's lane offsets span one Z block (S*128 bytes) and a slab
  if (lay.n_slots() * 128 + 8192 >= (1LL << 31)) return hipErrorInvalidConfiguration;
  // whole rounds on the wide configuration, a last round of <= cus/2 tiles as halves
  if (cus < 2) cus = 2;
  const long long rem = tiles % cus;
  const long long whole = rem <= cus / 2 ? tiles - rem : tiles;
  UpdArgs p{Z, VT, state_in, state_out, snap, W0p, lay.n_slots(), lay.L, lay.d, lay.f, 0, launch_round(cus),
            lay.seqs()};
  if (whole > 0) hipLaunchKernelGGL((k_update<WN_W, NBJ_W, NSL_W>), dim3((unsigned)whole), dim3(NT_W), 0, s, p);
  if (tiles > whole) {
    p.tile0 = (int)whole;
    hipLaunchKernelGGL((k_update<WN_U, NBJ_U, NSL_U>), dim3((unsigned)(2 * (tiles - whole))), dim3(NT_U), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_scores_bf16(const bf16_t *Z, bf16_t *P, const Layout &lay, int cus, hipStream_t s) {
  const int nt = (lay.L + 255) / 256;
  ScoreArgs p{Z, P, lay.n_slots(), lay.L, lay.C, lay.f, nt, launch_round(cus), lay.seqs(), 0, {}, {}};
  if (nt * (nt + 1) / 2 <= kMaxScorePairs) {
    // with C = 128 and an even number of tiles, the diagonal tiles go in packed pairs
    const bool pack = lay.C == 128 && lay.L % 512 == 0;
    // the tiles of a full group that the kernel would not skip, jt-major
    for (int jt = 0; jt < nt; ++jt) {
      const int jl = (jt * 256 + 255 < lay.L - 1) ? jt * 256 + 255 : lay.L - 1;
      for (int it = 0; it <= jt; ++it)
        if (it * 256 / lay.C < jl / lay.C && !(pack && it == jt)) {
          p.pit[p.npairs] = (unsigned char)it;
          p.pjt[p.npairs] = (unsigned char)jt;
          ++p.npairs;
        }
    }
    for (int a = 0; pack && a < nt; a += 2) {
      p.pit[p.npairs] = kPackedPair;
      p.pjt[p.npairs] = (unsigned char)a;
      ++p.npairs;
    }
    if (p.npairs == 0) return hipSuccess;  // one chunk per group: no within-group term
  }
  const long long n = lay.n_groups() * (p.npairs > 0 ? p.npairs : nt * (nt + 1) / 2);
  if (n >= (1LL << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_scores, dim3((unsigned)n), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_state_to_snap_bf16(const float *W0, const float *D, bf16_t *snap, int d, int f, hipStream_t s) {
  if (d <= 0 || f <= 0 || f % 8) return hipErrorInvalidValue;
  const long long n = (long long)d * (f / 8);
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_state_to_snap, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s, W0, D, snap,
                     d, f);
  return hipGetLastError();
}

hipError_t launch_to_planes_bf16(const bf16_t *src, bf16_t *dst, int d, int f, hipStream_t s) {
  if (d <= 0 || f <= 0 || f % 8) return hipErrorInvalidValue;
  const long long n = (long long)d * (f / 8);
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_to_planes, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s, src, dst, d, f);
  return hipGetLastError();
}

hipError_t launch_out_bf16(const bf16_t *Z, const bf16_t *P, const bf16_t *snap, const bf16_t *VT, void *y,
                           int y_f32, const Layout &lay, int cus, hipStream_t s) {
  OutArgs p{Z, P, snap, VT, y, lay.n_slots(), lay.L, lay.C, lay.d, lay.f, lay.intra, y_f32, launch_round(cus),
            lay.seqs()};
  const long long n = lay.n_groups() * (lay.d / BM) * ((lay.L + 255) / 256);
  if (n >= (1LL << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_out, dim3((unsigned)n), dim3(NT_W), 0, s, p);
  return hipGetLastError();
}
