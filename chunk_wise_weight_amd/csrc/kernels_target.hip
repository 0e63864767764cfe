// The general LM-aligned target V^ = Conv1D(X0) W_target (paperlayer.ai
// summary, sec. 3 "LM-Aligned Objective"; iplexlaw.co.kr walkthrough, sec. 4
// and sec. 6): a depthwise convolution of K taps over the token embeddings on
// the tokens after each position, then a d x d projection.
//
// Row t of chunk i (chunks of C counted from the call's first token) sums
// tap k on the embedding of the token at position t+1+k only while that
// position is at most min((i+1)C, T): the chunk boundary pads the
// convolution, except for the first token of the next chunk, which that chunk
// already holds as its input. With K = 1, weight 1 and W_target = I this is
// the next-token gather.
#include "launch.h"

namespace {

template <typename Tin>
__device__ __forceinline__ float to_f32(Tin v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

// 8 consecutive elements of a row, loaded at once (16-byte aligned for bf16,
// 32-byte aligned for fp32: a0 and d are multiples of 8); v(j) converts
// element j as to_f32 does.
template <typename Tv>
struct Row;
template <>
struct Row<bf16_t> {
  uint4 q;
  __device__ __forceinline__ float v(int j) const {
    const uint32_t w = (&q.x)[j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Row<float> {
  float4 lo, hi;
  __device__ __forceinline__ float v(int j) const { return j < 4 ? (&lo.x)[j] : (&hi.x)[j - 4]; }
};
__device__ __forceinline__ Row<bf16_t> load_row8(const bf16_t *p) {
  Row<bf16_t> r;
  r.q = *reinterpret_cast<const uint4 *>(p);
  return r;
}
__device__ __forceinline__ Row<float> load_row8(const float *p) {
  Row<float> r;
  r.lo = *reinterpret_cast<const float4 *>(p);
  r.hi = *reinterpret_cast<const float4 *>(p + 4);
  return r;
}

__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t *p, float v) { *p = f32_to_bf16(v); }

// U[slot][a] = sum_k cw[k][a] * E[ids of position t+1+k][a] (fp32 sums) for
// position t of the slot's sequence (its ids at SeqInfo::id0), rows past the
// sequence's length zero. One thread per (slot, group of 8 model dims).
template <typename Tv>
__global__ __launch_bounds__(256) void k_conv_taps(const int32_t *ids, const Tv *E, int vocab, const float *cw, int K,
                                                   Tv *U, Seqs sq, int C, int d, long long ngroups8) {
  for (long long g = (long long)blockIdx.x * 256 + threadIdx.x; g < ngroups8; g += (long long)gridDim.x * 256) {
    const int a0 = (int)(g % (d / 8)) * 8;
    const long long slot = g / (d / 8);
    const SeqInfo si = sq.at(sq.of_tile((int)(slot / 256)));
    const int t = (int)(slot - si.slot0), T = si.len;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t < T) {
      const long long chunk_end = ((long long)(t / C) + 1) * C;
      const int limit = (int)(chunk_end < T ? chunk_end : T);
      for (int k = 0; k < K; ++k) {
        const int p = t + 1 + k;
        if (p > limit) break;
        const int tok = ids[si.id0 + p];
        if (tok < 0 || tok >= vocab) continue;
        const Tv *e = E + (long long)tok * d + a0;
        const float *w = cw + (long long)k * d + a0;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += w[j] * to_f32(e[j]);
      }
    }
    Tv *u = U + slot * d + a0;
#pragma unroll
    for (int j = 0; j < 8; ++j) store_out(u + j, acc[j]);
  }
}

// The same sums for KT <= 8 taps, R consecutive slots per thread: the R+KT-1
// rows the run touches are read once each (instead of KT times) and added,
// in tap order, into every slot whose window holds them. Same arithmetic and
// order per slot as k_conv_taps, so the same results.
template <typename Tv, int KT>
__global__ __launch_bounds__(256) void k_conv_taps_run(const int32_t *ids, const Tv *E, int vocab, const float *cw,
                                                       Tv *U, Seqs sq, int C, int d, long long nthreads) {
  constexpr int R = 8;
  for (long long g = (long long)blockIdx.x * 256 + threadIdx.x; g < nthreads; g += (long long)gridDim.x * 256) {
    const int a0 = (int)(g % (d / 8)) * 8;
    const long long slot0 = g / (d / 8) * R;  // a run never straddles two sequences (their slots are 256-aligned)
    const SeqInfo si = sq.at(sq.of_tile((int)(slot0 / 256)));
    const int t0 = (int)(slot0 - si.slot0), T = si.len;
    float w[KT][8];
#pragma unroll
    for (int k = 0; k < KT; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) w[k][j] = cw[(long long)k * d + a0 + j];
    int limit[R];  // last position slot t0+r may take a tap from (its chunk's end, at most T); -1 past T
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const long long chunk_end = ((long long)((t0 + r) / C) + 1) * C;
      limit[r] = t0 + r < T ? (int)(chunk_end < T ? chunk_end : T) : -1;
    }
    float acc[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[r][j] = 0.f;
    // Window row i sits at position t0 + 1 + i; slot t0+r takes it as tap i-r.
    // All ids are loaded first and then all rows, so the loads overlap
    // instead of waiting one id and one row at a time; a row past T or with
    // an id outside [0, vocab) is read from row 0 and left out of the sums.
    constexpr int NW = R + KT - 1;
    int tok[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int p = t0 + 1 + i;
      tok[i] = p <= T ? ids[si.id0 + p] : -1;
    }
    bool ok[NW];
    Row<Tv> ev[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      ok[i] = tok[i] >= 0 && tok[i] < vocab;
      ev[i] = load_row8(E + (long long)(ok[i] ? tok[i] : 0) * d + a0);
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      if (!ok[i]) continue;
      const int p = t0 + 1 + i;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int k = i - r;
        if (k < 0 || k >= KT || p > limit[r]) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r][j] += w[k][j] * ev[i].v(j);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      Tv *u = U + (slot0 + r) * d + a0;
#pragma unroll
      for (int j = 0; j < 8; ++j) store_out(u + j, acc[r][j]);
    }
  }
}

// fp32 path: VT[b][a][t] = sum_c U[b][t][c] W[c][a]; Vrow[b][t][a] the same value (optional).
__global__ __launch_bounds__(256) void k_target_gemm_f32(const float *U, const float *W, float *VT, float *Vrow,
                                                         int T_pad, int d, long long n) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const int t = (int)(e % T_pad);
    const long long ba = e / T_pad;
    const int a = (int)(ba % d);
    const int b = (int)(ba / d);
    const float *u = U + ((long long)b * T_pad + t) * d;
    float s = 0.f;
    for (int c = 0; c < d; ++c) s += u[c] * W[(long long)c * d + a];
    VT[e] = s;
    if (Vrow) Vrow[((long long)b * T_pad + t) * d + a] = s;
  }
}

// dst[j][i] = src[i][j] for an n x n matrix (set-up only).
template <typename Tv>
__global__ __launch_bounds__(256) void k_transpose(const Tv *src, Tv *dst, int n) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < (long long)n * n; e += (long long)gridDim.x * 256) {
    const int i = (int)(e / n), j = (int)(e % n);
    dst[(long long)j * n + i] = src[e];
  }
}

__global__ __launch_bounds__(256) void k_copy_f32(const float *src, float *dst, long long n) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) dst[e] = src[e];
}

unsigned grid_for(long long n) {
  long long g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

template <typename Tv, int KT>
hipError_t launch_conv_run(const int32_t *ids, const Tv *E, int vocab, const float *cw, Tv *U, const Layout &lay,
                           hipStream_t s) {
  const long long n = lay.n_slots() / 8 * (lay.d / 8);
  hipLaunchKernelGGL((k_conv_taps_run<Tv, KT>), dim3(grid_for(n)), dim3(256), 0, s, ids, E, vocab, cw, U, lay.seqs(),
                     lay.C, lay.d, n);
  return hipGetLastError();
}

// Runs of 8 slots for up to 8 taps, one slot per thread beyond.
template <typename Tv>
hipError_t launch_conv_taps(const int32_t *ids, const Tv *E, int vocab, const float *cw, int K, Tv *U,
                            const Layout &lay, hipStream_t s) {
  switch (K) {
    case 1: return launch_conv_run<Tv, 1>(ids, E, vocab, cw, U, lay, s);
    case 2: return launch_conv_run<Tv, 2>(ids, E, vocab, cw, U, lay, s);
    case 3: return launch_conv_run<Tv, 3>(ids, E, vocab, cw, U, lay, s);
    case 4: return launch_conv_run<Tv, 4>(ids, E, vocab, cw, U, lay, s);
    case 5: return launch_conv_run<Tv, 5>(ids, E, vocab, cw, U, lay, s);
    case 6: return launch_conv_run<Tv, 6>(ids, E, vocab, cw, U, lay, s);
    case 7: return launch_conv_run<Tv, 7>(ids, E, vocab, cw, U, lay, s);
    case 8: return launch_conv_run<Tv, 8>(ids, E, vocab, cw, U, lay, s);
    default: break;
  }
  const long long n = lay.n_slots() * (lay.d / 8);
  hipLaunchKernelGGL((k_conv_taps<Tv>), dim3(grid_for(n)), dim3(256), 0, s, ids, E, vocab, cw, K, U, lay.seqs(), lay.C,
                     lay.d, n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_taps_bf16(const int32_t *ids, const bf16_t *E, int vocab, const float *cw, int K, bf16_t *U,
                                 const Layout &lay, hipStream_t s) {
  return launch_conv_taps<bf16_t>(ids, E, vocab, cw, K, U, lay, s);
}

hipError_t launch_conv_taps_f32(const int32_t *ids, const float *E, int vocab, const float *cw, int K, float *U,
                                const Layout &lay, hipStream_t s) {
  return launch_conv_taps<float>(ids, E, vocab, cw, K, U, lay, s);
}

hipError_t launch_target_gemm_f32(const float *U, const float *W, float *VT, float *Vrow, const Layout &lay,
                                  hipStream_t s) {
  const long long n = (long long)lay.B * lay.d * lay.T_pad;
  hipLaunchKernelGGL(k_target_gemm_f32, dim3(grid_for(n)), dim3(256), 0, s, U, W, VT, Vrow, lay.T_pad, lay.d, n);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const bf16_t *src, bf16_t *dst, int n, hipStream_t s) {
  hipLaunchKernelGGL((k_transpose<bf16_t>), dim3(grid_for((long long)n * n)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float *src, float *dst, long long n, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_f32, dim3(grid_for(n)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}
