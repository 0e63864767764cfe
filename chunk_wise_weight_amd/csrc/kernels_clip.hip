// Frobenius-norm clipping of each chunk update (paperlayer.ai summary,
// App. C.2 "Inference Stability"; iplexlaw.co.kr walkthrough, sec. 6): before
// chunk i's update dW_i = eta V_i^T Z_i is applied it is rescaled by
// c_i = min(1, tau / ||dW_i||_F). Scaling the chunk's target rows V_i by c_i
// applies the clip everywhere the update enters: the state update
// (sum_i c_i eta V_i^T Z_i) and the within-group term of the outputs
// (P[t][s] V[s] with V[s] scaled by the factor of s's chunk).
//
// The squared norm comes from the chunk Grams, ||V_i^T Z_i||_F^2 =
// sum_{s,t in chunk i} <v_s, v_t> <z_s, z_t>, taken per row s into `rowpart`
// (the MFMA kernel on the bf16 path, the plain kernel below on the fp32 path)
// and summed here per chunk in a fixed order.
#include "launch.h"

namespace {

// rowpart[slot/256][wr][slot%256] summed over wr and the chunk's rows (slots
// of sequence b: its own chunks, counted from its first position); one
// workgroup per (chunk, sequence); c[b][i] = min(1, tau / (|eta| sqrt(sum))),
// 1 for a chunk past the sequence's end.
__global__ __launch_bounds__(256) void k_chunk_factors(const float *rowpart, float *cfac, Seqs sq, int C, int wspan,
                                                       int nchunks, float eta, float tau) {
  __shared__ float red[256];
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const SeqInfo si = sq.at(b);
  const long long c0 = (long long)i * C;
  const long long c1 = (long long)(i + 1) * C < si.len ? (long long)(i + 1) * C : si.len;
  float sum = 0.f;
  for (long long s = c0 + tid; s < c1; s += 256) {
    const long long slot = si.slot0 + s;
    const float *rp = rowpart + ((slot / 256) * wspan) * 256 + slot % 256;
    for (int wr = 0; wr < wspan; ++wr) sum += rp[wr * 256];
  }
  red[tid] = sum;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  if (tid == 0) {
    const float n = fabsf(eta) * sqrtf(fmaxf(red[0], 0.f));
    cfac[(long long)b * nchunks + i] = n > tau ? tau / n : 1.f;
  }
}

// V^T K-blocked [S/64][d][64] (bf16): the slot at position p of sequence b
// scaled by c[b][p / C]; slots past the sequence's length are zero and stay
// so. 8 elements (8 slots of one model dim, one 64-slot block) per thread.
__global__ __launch_bounds__(256) void k_scale_vt_bf16(bf16_t *VT, const float *cfac, Seqs sq, int C, int d,
                                                       int nchunks, long long n8) {
  for (long long g = (long long)blockIdx.x * 256 + threadIdx.x; g < n8; g += (long long)gridDim.x * 256) {
    const long long e = g * 8;
    const long long slot = e / ((long long)d * 64) * 64 + e % 64;  // the first of the 8
    const int b = sq.of_tile((int)(slot / 256));
    const SeqInfo si = sq.at(b);
    const int p0 = (int)(slot - si.slot0), T = si.len;
    if (p0 >= T) continue;
    uint4 raw = *reinterpret_cast<const uint4 *>(VT + e);
    bf16_t *v = reinterpret_cast<bf16_t *>(&raw);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = p0 + k;
      if (t < T) v[k] = f32_to_bf16(bf16_to_f32(v[k]) * cfac[(long long)b * nchunks + t / C]);
    }
    *reinterpret_cast<uint4 *>(VT + e) = raw;
  }
}

// V^T row-major [B][d][T_pad] (fp32): column t of sequence b scaled by c[b][t / C].
__global__ __launch_bounds__(256) void k_scale_vt_f32(float *VT, const float *cfac, int T, int T_pad, int C, int d,
                                                      int nchunks, long long n) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const int t = (int)(e % T_pad);
    if (t >= T) continue;
    const int b = (int)(e / ((long long)d * T_pad));
    VT[e] *= cfac[(long long)b * nchunks + t / C];
  }
}

// fp32 path: rowpart[b][s] = sum over t in s's chunk of <v_s, v_t> <z_s, z_t>
// (the layout of the MFMA kernel's rowpart with one t-tile per row group).
// One workgroup per (row, sequence); plain fp32 dot products.
__global__ __launch_bounds__(256) void k_chunk_gram_f32(const float *Z, const float *V, float *rowpart, int T,
                                                        int T_pad, int C, int d, int f) {
  __shared__ float red[256];
  const int s = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  float sum = 0.f;
  if (s < T) {
    const long long c0 = (long long)(s / C) * C;
    const long long c1 = c0 + C < T ? c0 + C : T;
    const float *zs = Z + ((long long)b * T_pad + s) * f;
    const float *vs = V + ((long long)b * T_pad + s) * d;
    for (long long t = c0 + tid; t < c1; t += 256) {
      const float *zt = Z + ((long long)b * T_pad + t) * f;
      const float *vt = V + ((long long)b * T_pad + t) * d;
      float gz = 0.f, gv = 0.f;
      for (int k = 0; k < f; ++k) gz += zs[k] * zt[k];
      for (int k = 0; k < d; ++k) gv += vs[k] * vt[k];
      sum += gz * gv;
    }
  }
  red[tid] = sum;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  if (tid == 0) rowpart[(long long)b * T_pad + s] = red[0];
}

unsigned grid_for(long long n) {
  long long g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

// The most 256-token t-tiles that hold a token sharing a chunk with some token
// of one 256-token s-tile, over the s-tiles of the stream: the bf16 Gram
// kernel's t-tiles per s-tile, so its grid has no slot without work when every
// s-tile needs as many (chunk sizes dividing 256, or multiples of it).
int clip_wspan(const Layout &lay, bool bf16) {
  if (!bf16) return 1;
  const long long C = lay.C, T = lay.T, nw = lay.T_pad / 256;
  long long best = 1;
  for (long long s0 = 0; s0 < T; s0 += 256) {
    const long long s_last = s0 + 255 < T - 1 ? s0 + 255 : T - 1;
    const long long w_lo = (s0 / C) * C / 256;
    long long w_hi = ((s_last / C + 1) * C - 1) / 256;
    if (w_hi > nw - 1) w_hi = nw - 1;
    if (w_hi - w_lo + 1 > best) best = w_hi - w_lo + 1;
  }
  return (int)best;
}

size_t clip_gram_scratch_bytes(const Layout &lay, int wspan) {
  return (size_t)(lay.n_slots() / 256) * wspan * (256 * 256 * 4);
}

// chunks per sequence in the factor table c[sequence][chunk]: those of the
// caller's T (no sequence is longer)
int clip_chunks(const Layout &lay) { return (int)((lay.T + (long long)lay.C - 1) / lay.C); }

hipError_t launch_chunk_factors(const float *rowpart, float *cfac, int wspan, float eta, float tau, const Layout &lay,
                                hipStream_t s) {
  const int nchunks = clip_chunks(lay);
  hipLaunchKernelGGL(k_chunk_factors, dim3(nchunks, lay.n_seq()), dim3(256), 0, s, rowpart, cfac, lay.seqs(), lay.C,
                     wspan, nchunks, eta, tau);
  return hipGetLastError();
}

hipError_t launch_scale_vt_bf16(bf16_t *VT, const float *cfac, const Layout &lay, hipStream_t s) {
  const long long n8 = lay.n_slots() * lay.d / 8;
  hipLaunchKernelGGL(k_scale_vt_bf16, dim3(grid_for(n8)), dim3(256), 0, s, VT, cfac, lay.seqs(), lay.C, lay.d,
                     clip_chunks(lay), n8);
  return hipGetLastError();
}

hipError_t launch_scale_vt_f32(float *VT, const float *cfac, const Layout &lay, hipStream_t s) {
  const long long n = (long long)lay.B * lay.d * lay.T_pad;
  hipLaunchKernelGGL(k_scale_vt_f32, dim3(grid_for(n)), dim3(256), 0, s, VT, cfac, lay.T, lay.T_pad, lay.C, lay.d,
                     clip_chunks(lay), n);
  return hipGetLastError();
}

hipError_t launch_chunk_gram_f32(const float *Z, const float *Vrow, float *rowpart, const Layout &lay, hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_gram_f32, dim3(lay.T_pad, lay.B), dim3(256), 0, s, Z, Vrow, rowpart, lay.T, lay.T_pad,
                     lay.C, lay.d, lay.f);
  return hipGetLastError();
}
