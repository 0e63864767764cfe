// MFMA throughput and shader clock under the chip's power limit.
//
// Every compute unit runs only bf16 MFMAs (no memory traffic in the timed
// loop) on random operands that alternate between two register sets, in one
// of two shapes with the same work per cycle: v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_16x16x32_bf16, each wave on a 128 x 64 tile of accumulators,
// with 8 or 4 waves per compute unit. It prints the achieved rate (HIP events)
// and the shader clock each workgroup saw (s_memtime, which counts shader
// clocks, against s_memrealtime, which counts the constant wall clock), and
// the rate as a fraction of the peak at that clock (1024 flop per clock per
// SIMD, 4 SIMDs per compute unit).
//
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops mfma_clock.hip
// Run:   ./mfma_clock [iterations]
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                       \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      std::exit(1);                                                                    \
    }                                                                                  \
  } while (0)

constexpr int kPerLane = 24;  // bf16x8 operands per lane in the input table

// SHAPE 32: 4 x 2 accumulators of 32 x 32, two 16-deep k steps per iteration.
// SHAPE 16: 8 x 4 accumulators of 16 x 16, two 32-deep k steps per iteration.
template <int SHAPE>
__global__ __launch_bounds__(512) void burn(const bf16x8 *in, float *out, int iters, unsigned long long *clk) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[2][8], b[2][4];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[k][i] = in[lane * kPerLane + k * 12 + i];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[k][j] = in[lane * kPerLane + k * 12 + 8 + j];
  }
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  float s = 0.f;
  if constexpr (SHAPE == 32) {
    f32x16 acc[4][2] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int bj = 0; bj < 2; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k][bi + 4 * bj], b[k][bj + 2 * (bi & 1)],
                                                                  acc[bi][bj], 0, 0, 0);
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[bi][bj][e];
  } else {
    f32x4 acc[8][4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int bi = 0; bi < 8; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k][bi], b[k][bj], acc[bi][bj], 0, 0, 0);
    }
#pragma unroll
    for (int bi = 0; bi < 8; ++bi)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += acc[bi][bj][e];
  }
  if (threadIdx.x == 0) {
    clk[blockIdx.x * 4 + 0] = t0;
    clk[blockIdx.x * 4 + 1] = __builtin_amdgcn_s_memtime();
    clk[blockIdx.x * 4 + 2] = r0;
    clk[blockIdx.x * 4 + 3] = __builtin_amdgcn_s_memrealtime();
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the MFMAs live
}

template <int SHAPE>
void run(const bf16x8 *din, float *dout, unsigned long long *dclk, int cus, int block, int iters, double wall_khz) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL(burn<SHAPE>, dim3(cus), dim3(block), 0, 0, din, dout, iters / 10, dclk);  // warm-up
  CHECK(hipDeviceSynchronize());
  for (int rep = 0; rep < 3; ++rep) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(burn<SHAPE>, dim3(cus), dim3(block), 0, 0, din, dout, iters, dclk);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::vector<unsigned long long> c((size_t)cus * 4);
    CHECK(hipMemcpy(c.data(), dclk, c.size() * 8, hipMemcpyDeviceToHost));
    double ratio = 0;
    for (int g = 0; g < cus; ++g)
      ratio += double(c[g * 4 + 1] - c[g * 4]) / double(c[g * 4 + 3] - c[g * 4 + 2]);
    const double ghz = ratio / cus * wall_khz * 1e-6;
    const double flop = 2.0 * 128 * 64 * (SHAPE == 32 ? 32 : 64) * (double)iters * cus * (block / 64);
    const double tflops = flop / ms * 1e-9;
    const double peak = 4.0 * 1024 * cus * ghz * 1e-3;  // TFLOP/s at that clock
    std::printf("%-10s %2d waves/CU  %8.3f ms  %7.1f TFLOP/s  shader clock %.3f GHz  %5.1f%% of the peak at that clock\n",
                SHAPE == 32 ? "32x32x16" : "16x16x32", block / 64, ms, tflops, ghz, 100.0 * tflops / peak);
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

int main(int argc, char **argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 100000;
  int wall_khz = 0, cus = 0;
  CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  std::printf("compute units %d, wall clock %d kHz, %d iterations (half as many for 16x16x32, whose iteration is twice "
              "the work)\n",
              cus, wall_khz, iters);
  const int n = 64 * kPerLane * 8;
  std::vector<uint16_t> h(n);
  std::srand(1);
  for (int i = 0; i < n; ++i) {
    const float v = (std::rand() / (float)RAND_MAX) * 2.f - 1.f;
    uint32_t u;
    std::memcpy(&u, &v, 4);
    h[i] = (uint16_t)(u >> 16);
  }
  bf16x8 *din;
  float *dout;
  unsigned long long *dclk;
  CHECK(hipMalloc(&din, n * 2));
  CHECK(hipMalloc(&dout, (size_t)cus * 512 * 4));
  CHECK(hipMalloc(&dclk, (size_t)cus * 4 * 8));
  CHECK(hipMemcpy(din, h.data(), n * 2, hipMemcpyHostToDevice));
  run<32>(din, dout, dclk, cus, 512, iters, wall_khz);
  run<16>(din, dout, dclk, cus, 512, iters / 2, wall_khz);
  run<32>(din, dout, dclk, cus, 256, iters, wall_khz);
  run<16>(din, dout, dclk, cus, 256, iters / 2, wall_khz);
  CHECK(hipFree(din));
  CHECK(hipFree(dout));
  CHECK(hipFree(dclk));
  return 0;
}
