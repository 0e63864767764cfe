// Layout and conversion helpers used at init, reset and for the eta = 0 case.
#include "launch.h"

namespace {

// Wug row r: block r/64; rows 0..31 of a block are W_up rows 32*(r/64)+..., rows 32..63 the matching W_gate rows.
__global__ __launch_bounds__(256) void k_interleave_ug(const bf16_t *Wu, const bf16_t *Wg, bf16_t *Wug, int f, int d) {
  const int r = blockIdx.x;
  const int blk = r >> 6, w = r & 63;
  const bf16_t *src = (w < 32 ? Wu : Wg) + (long long)(blk * 32 + (w & 31)) * d;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8)
    *reinterpret_cast<uint4 *>(Wug + ((long long)(c / 64) * 2 * f + r) * 64 + c % 64) =
        *reinterpret_cast<const uint4 *>(src + c);
}

__global__ __launch_bounds__(256) void k_bf16_to_f32(const bf16_t *src, float *dst, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    dst[i] = bf16_to_f32(src[i]);
}

__global__ __launch_bounds__(256) void k_fill_f32(float *dst, float v, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) dst[i] = v;
}

// out[b][k] = W0[k] + D[b][k], four elements per thread step (n a multiple of 4)
__global__ __launch_bounds__(256) void k_add_state(const float *W0, const float *D, float *out, int B, long long n4) {
  const long long total = (long long)B * n4;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const float4 w = reinterpret_cast<const float4 *>(W0)[i % n4];
    const float4 d = reinterpret_cast<const float4 *>(D)[i];
    reinterpret_cast<float4 *>(out)[i] = make_float4(w.x + d.x, w.y + d.y, w.z + d.z, w.w + d.w);
  }
}

unsigned grid_for(long long n) {
  long long g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

hipError_t launch_interleave_ug_bf16(const bf16_t *Wu, const bf16_t *Wg, bf16_t *Wug, int f, int d, hipStream_t s) {
  hipLaunchKernelGGL(k_interleave_ug, dim3(2 * f), dim3(256), 0, s, Wu, Wg, Wug, f, d);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f32(const bf16_t *src, float *dst, long long n, hipStream_t s) {
  hipLaunchKernelGGL(k_bf16_to_f32, dim3(grid_for(n)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}


hipError_t launch_fill_f32(float *dst, float v, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(n)), dim3(256), 0, s, dst, v, n);
  return hipGetLastError();
}

hipError_t launch_add_state_f32(const float *W0, const float *D, float *out, int B, long long n, hipStream_t s) {
  if (B <= 0 || n <= 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_add_state, dim3(grid_for((long long)B * n / 4)), dim3(256), 0, s, W0, D, out, B, n / 4);
  return hipGetLastError();
}
