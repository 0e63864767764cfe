// fp32 kernels of the chunk-wise fast-weight path (plain FMA, gfx950).
//
// Same buffers, layouts and two-level scan as the bf16 MFMA path, computed in
// fp32 end to end. A block computes a 64 x 64 tile D[i][j] = sum_k A[i][k] B[j][k]
// with 256 threads (4 x 4 outputs each); k advances 16 at a time through LDS.
#include "launch.h"

namespace {

constexpr int TM = 64, TN = 64, TK = 16, NT = 256;

typedef float Tile[TK][TM + 4];

struct AccF {
  float v[4][4];  // [j offset][i offset]: four consecutive i for each j
};

__device__ __forceinline__ void accf_zero(AccF &a) {
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) a.v[x][y] = 0.f;
}

// rows [row0, row0+64) x cols [k, k+16) of a segment, stored k-major in LDS
__device__ __forceinline__ void tile_load(Tile &t, const Seg<float> &s, int row0, int k, int tid) {
  const int r = tid >> 2, kc = (tid & 3) * 4;
  const int row = row0 + r, kk = k + kc;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (row < s.nrows && kk < s.kvalid) v = *reinterpret_cast<const float4 *>(s.base + (long long)row * s.ld + kk);
  t[kc + 0][r] = v.x;
  t[kc + 1][r] = v.y;
  t[kc + 2][r] = v.z;
  t[kc + 3][r] = v.w;
}

__device__ __forceinline__ void tile_fma(AccF &acc, const Tile &A, const Tile &B, int k, int tx, int ty) {
  const float4 a = *reinterpret_cast<const float4 *>(&A[k][tx * 4]);
  const float4 b = *reinterpret_cast<const float4 *>(&B[k][ty * 4]);
  const float av[4] = {a.x, a.y, a.z, a.w};
  const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int y = 0; y < 4; ++y)
#pragma unroll
    for (int x = 0; x < 4; ++x) acc.v[y][x] = fmaf(av[x], bv[y], acc.v[y][x]);
}

__device__ void simt_loop(AccF &acc, Tile &As, Tile &Bs, const Seg<float> &a1, const Seg<float> &b1, int nk1,
                          const Seg<float> &a2, const Seg<float> &b2, int nk2, int arow0, int brow0) {
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  for (int kt = 0; kt < nk1 + nk2; ++kt) {
    if (kt < nk1) {
      tile_load(As, a1, arow0, kt * TK, tid);
      tile_load(Bs, b1, brow0, kt * TK, tid);
    } else {
      tile_load(As, a2, arow0, (kt - nk1) * TK, tid);
      tile_load(Bs, b2, brow0, (kt - nk1) * TK, tid);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) tile_fma(acc, As, Bs, k, tx, ty);
    __syncthreads();
  }
}

// Up/gate GEMM + SwiGLU. i = token slot, j = hidden unit. grid (ceil(f/64), B*T_pad/64)
__global__ __launch_bounds__(NT) void k_a1_f32(const float *x, const float *Wu, const float *Wg, float *Z, float *ZT,
                                               float eta, int write_zt, int T, int T_pad, int d, int f) {
  __shared__ __attribute__((aligned(16))) Tile As, Bu, Bg;
  const int n0 = blockIdx.x * TN, m0 = blockIdx.y * TM;
  const int b = m0 / T_pad, pos0 = m0 - b * T_pad;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  Seg<float> sa{x + ((long long)b * T + pos0) * d, d, T - pos0, d};
  Seg<float> su{Wu, d, f, d}, sg{Wg, d, f, d};
  AccF au, ag;
  accf_zero(au);
  accf_zero(ag);
  for (int k = 0; k < d; k += TK) {
    tile_load(As, sa, 0, k, tid);
    tile_load(Bu, su, n0, k, tid);
    tile_load(Bg, sg, n0, k, tid);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      tile_fma(au, As, Bu, kk, tx, ty);
      tile_fma(ag, As, Bg, kk, tx, ty);
    }
    __syncthreads();
  }
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int feat = n0 + ty * 4 + y;
    if (feat >= f) continue;
    const int pos = pos0 + tx * 4;
    float z[4];
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) {
      const float g = ag.v[y][xx];
      z[xx] = g / (1.0f + expf(-g)) * au.v[y][xx];
      Z[((long long)b * T_pad + pos + xx) * f + feat] = z[xx];
    }
    if (write_zt)
      *reinterpret_cast<float4 *>(ZT + ((long long)b * f + feat) * T_pad + pos) =
          make_float4(eta * z[0], eta * z[1], eta * z[2], eta * z[3]);
  }
}

// State update with fp32 snapshots at every group start. i = hidden unit, j = model dim.
// grid (ceil(f/64), ceil(d/64), B)
// The state is D = W - W0 (the change since the last reset); snapshots are W0 + D.
__global__ __launch_bounds__(NT) void k_update_f32(const float *ZT, const float *VT, float *state, float *snap,
                                                   const float *W0, int T_pad, int kend, int L, int ngroups, int d,
                                                   int f) {
  __shared__ __attribute__((aligned(16))) Tile As, Bs;
  const int i0 = blockIdx.x * TM, j0 = blockIdx.y * TN, b = blockIdx.z;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float *st = state + (long long)b * d * f;
  float *sn = snap + (long long)b * ngroups * d * f;
  // The accumulators carry D, which starts at zero after a reset and stays
  // small next to W: increments far below the fp32 resolution of W itself (as
  // with clipped updates) still accumulate with fp32 relative precision. W0
  // stays in registers and is added for each snapshot.
  AccF acc, w0;
  const int i = i0 + tx * 4;
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int a = j0 + ty * 4 + y;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f), u = v;
    if (a < d && i < f) {
      v = *reinterpret_cast<const float4 *>(st + (long long)a * f + i);
      u = *reinterpret_cast<const float4 *>(W0 + (long long)a * f + i);
    }
    acc.v[y][0] = v.x;
    acc.v[y][1] = v.y;
    acc.v[y][2] = v.z;
    acc.v[y][3] = v.w;
    w0.v[y][0] = u.x;
    w0.v[y][1] = u.y;
    w0.v[y][2] = u.z;
    w0.v[y][3] = u.w;
  }
  auto dump = [&](int g) {
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int a = j0 + ty * 4 + y;
      if (a < d && i < f)
        *reinterpret_cast<float4 *>(sn + ((long long)g * d + a) * f + i) =
            make_float4(w0.v[y][0] + acc.v[y][0], w0.v[y][1] + acc.v[y][1], w0.v[y][2] + acc.v[y][2],
                        w0.v[y][3] + acc.v[y][3]);
    }
  };
  Seg<float> sa{ZT + (long long)b * f * T_pad, T_pad, f, T_pad};
  Seg<float> sb{VT + (long long)b * d * T_pad, T_pad, d, T_pad};
  int g = 0;
  for (int k0 = 0; k0 < kend; k0 += TK) {
    tile_load(As, sa, i0, k0, tid);
    tile_load(Bs, sb, j0, k0, tid);
    __syncthreads();
    for (int kk = 0; kk < TK; ++kk) {
      while (g < ngroups && (long long)g * L == k0 + kk) dump(g++);
      tile_fma(acc, As, Bs, kk, tx, ty);
    }
    __syncthreads();
  }
  while (g < ngroups) dump(g++);
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int a = j0 + ty * 4 + y;
    if (a < d && i < f)
      *reinterpret_cast<float4 *>(st + (long long)a * f + i) =
          make_float4(acc.v[y][0], acc.v[y][1], acc.v[y][2], acc.v[y][3]);
  }
}

// Within-group scores, i = s, j = t, tiles with it <= jt. grid (nt*nt, ngroups, B)
__global__ __launch_bounds__(NT) void k_scores_f32(const float *Z, float *P, float eta, int T, int T_pad, int L,
                                                   int C, int ngroups, int f, int nt) {
  __shared__ __attribute__((aligned(16))) Tile As, Bs;
  const int it = blockIdx.x % nt, jt = blockIdx.x / nt, g = blockIdx.y, b = blockIdx.z;
  const long long gs = (long long)g * L;
  const int Lg = (int)((T - gs) < L ? (T - gs) : L);
  const int i0 = it * TM, j0 = jt * TN;
  if (it > jt || j0 >= Lg) return;
  const float *Zg = Z + ((long long)b * T_pad + gs) * f;
  Seg<float> s{Zg, f, (int)(T_pad - gs), f};
  AccF acc;
  accf_zero(acc);
  simt_loop(acc, As, Bs, s, s, f / TK, s, s, 0, i0, j0);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float *Pg = P + ((long long)b * ngroups + g) * L * L;
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int t = j0 + ty * 4 + y;
    const int sidx = i0 + tx * 4;
    if (t >= L || sidx >= L) continue;
    float v[4];
#pragma unroll
    for (int xx = 0; xx < 4; ++xx) v[xx] = ((sidx + xx) / C < t / C) ? eta * acc.v[y][xx] : 0.f;
    *reinterpret_cast<float4 *>(Pg + (long long)t * L + sidx) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Output: y[gL+t][a] = sum_k [snap | V^T][a][k] [Z | P][t][k]. i = a, j = t.
// grid (ceil(d/64), ceil(L/64), B*ngroups)
__global__ __launch_bounds__(NT) void k_out_f32(const float *Z, const float *P, const float *snap, const float *VT,
                                                float *y, int T, int T_pad, int L, int C, int ngroups, int d, int f,
                                                int intra) {
  __shared__ __attribute__((aligned(16))) Tile As, Bs;
  const int i0 = blockIdx.x * TM, j0 = blockIdx.y * TN;
  const int b = blockIdx.z / ngroups, g = blockIdx.z % ngroups;
  const long long gs = (long long)g * L;
  const int Lg = (int)((T - gs) < L ? (T - gs) : L);
  if (j0 >= Lg) return;
  Seg<float> a1{snap + ((long long)b * ngroups + g) * d * f, f, d, f};
  Seg<float> b1{Z + ((long long)b * T_pad + gs) * f, f, (int)(T_pad - gs), f};
  Seg<float> a2 = a1, b2 = b1;
  int nk2 = 0;
  if (intra) {
    const int jl = (j0 + TN - 1 < Lg - 1) ? j0 + TN - 1 : Lg - 1;
    const int kv = ((jl / C) * C + 7) & ~7;
    nk2 = (kv + TK - 1) / TK;
    a2 = Seg<float>{VT + (long long)b * d * T_pad + gs, T_pad, d, kv};
    b2 = Seg<float>{P + ((long long)b * ngroups + g) * L * L, L, L, kv};
  }
  AccF acc;
  accf_zero(acc);
  simt_loop(acc, As, Bs, a1, b1, f / TK, a2, b2, nk2, i0, j0);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int yy = 0; yy < 4; ++yy) {
    const int t = j0 + ty * 4 + yy;
    const int a = i0 + tx * 4;
    if (t >= Lg || a >= d) continue;
    *reinterpret_cast<float4 *>(y + ((long long)b * T + gs + t) * d + a) =
        make_float4(acc.v[yy][0], acc.v[yy][1], acc.v[yy][2], acc.v[yy][3]);
  }
}

// V^T[b][a][p] = E[ids[b][p+1]][a]. grid (T_pad/64, d/64, B)
__global__ __launch_bounds__(256) void k_gather_vt_f32(const int32_t *ids, const float *E, int vocab, float *VT,
                                                       float *Vrow, int T, int T_pad, int d) {
  __shared__ float tile[64][65];
  __shared__ int tok[64];
  const int p0 = blockIdx.x * 64, a0 = blockIdx.y * 64, b = blockIdx.z;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int pos = p0 + tid;
    tok[tid] = (pos < T) ? ids[(long long)b * (T + 1) + pos + 1] : -1;
  }
  __syncthreads();
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int pl = idx >> 6, a = idx & 63;
    const int id = tok[pl];
    const float v = (id >= 0 && id < vocab) ? E[(long long)id * d + a0 + a] : 0.f;
    tile[pl][a] = v;
    if (Vrow) Vrow[((long long)b * T_pad + p0 + pl) * d + a0 + a] = v;
  }
  __syncthreads();
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int al = idx >> 6, pl = idx & 63;
    VT[((long long)b * d + a0 + al) * T_pad + p0 + pl] = tile[pl][al];
  }
}

}  // namespace

hipError_t launch_gather_vt_f32(const int32_t *ids, const float *E, int vocab, float *VT, float *Vrow,
                                const Layout &lay, hipStream_t s) {
  dim3 grid(lay.T_pad / 64, lay.d / 64, lay.B);
  hipLaunchKernelGGL(k_gather_vt_f32, grid, dim3(256), 0, s, ids, E, vocab, VT, Vrow, lay.T, lay.T_pad, lay.d);
  return hipGetLastError();
}

hipError_t launch_a1_f32(const float *x, const float *Wug, float *Z, float *ZT, float eta, int write_zt,
                         const Layout &lay, hipStream_t s) {
  dim3 grid((lay.f + TN - 1) / TN, (unsigned)((long long)lay.B * lay.T_pad / TM));
  hipLaunchKernelGGL(k_a1_f32, grid, dim3(NT), 0, s, x, Wug, Wug + (long long)lay.f * lay.d, Z, ZT, eta, write_zt,
                     lay.T, lay.T_pad, lay.d, lay.f);
  return hipGetLastError();
}

hipError_t launch_update_f32(const float *ZT, const float *VT, float *state, float *snap, const float *W0,
                             const Layout &lay,
                             hipStream_t s) {
  const int kend = (int)round_up_ll(lay.T, TK);
  dim3 grid((lay.f + TM - 1) / TM, (lay.d + TN - 1) / TN, lay.B);
  hipLaunchKernelGGL(k_update_f32, grid, dim3(NT), 0, s, ZT, VT, state, snap, W0, lay.T_pad, kend, lay.L, lay.ngroups,
                     lay.d, lay.f);
  return hipGetLastError();
}

hipError_t launch_scores_f32(const float *Z, float *P, float eta, const Layout &lay, hipStream_t s) {
  const int nt = (lay.L + TN - 1) / TN;
  dim3 grid(nt * nt, lay.ngroups, lay.B);
  hipLaunchKernelGGL(k_scores_f32, grid, dim3(NT), 0, s, Z, P, eta, lay.T, lay.T_pad, lay.L, lay.C, lay.ngroups,
                     lay.f, nt);
  return hipGetLastError();
}

hipError_t launch_out_f32(const float *Z, const float *P, const float *snap, const float *VT, float *y,
                          const Layout &lay, hipStream_t s) {
  dim3 grid((lay.d + TM - 1) / TM, (lay.L + TN - 1) / TN, lay.B * lay.ngroups);
  hipLaunchKernelGGL(k_out_f32, grid, dim3(NT), 0, s, Z, P, snap, VT, y, lay.T, lay.T_pad, lay.L, lay.C, lay.ngroups,
                     lay.d, lay.f, lay.intra);
  return hipGetLastError();
}
