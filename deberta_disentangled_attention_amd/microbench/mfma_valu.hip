// Throughput of the gfx950 matrix unit alone and alongside transcendental
// VALU work, at 1, 2 and 4 waves per SIMD: the budget that the forward's
// far-tile loop (16 MFMAs and 32 exponentials per wave and key tile) runs in.
//
// Each wave runs a loop of NM independent 32x32x16 bf16 MFMAs (four
// accumulator chains) and NE exponential+multiply pairs (32 independent
// chains). The shader clock is read with s_memtime and calibrated against the
// 100 MHz s_memrealtime counter.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int NM, int NE>
__global__ __launch_bounds__(64) void loop_kernel(float* out, long long* clk, int iters, float seed) {
  f32x16 acc[4] = {};
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed + i);
  }
  float e[32];
  for (int i = 0; i < 32; ++i) e[i] = seed * (threadIdx.x + i) * 1e-3f;
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NE; ++i) e[i & 31] = __builtin_amdgcn_exp2f(e[i & 31]) * 0.5f;
  }
  const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 16; ++r) s += acc[m][r];
  for (int i = 0; i < 32; ++i) s += e[i];
  out[blockIdx.x * 64 + threadIdx.x] = s;   // keeps the work live
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)

template <int NM, int NE>
void run(const char* name, int waves_per_simd) {
  const int nblk = 1024 * waves_per_simd;   // 256 CUs x 4 SIMDs, one wave per block
  const int iters = 4000;
  float* out;
  long long* clk;
  CHECK(hipMalloc(&out, (size_t)nblk * 64 * sizeof(float)));
  CHECK(hipMalloc(&clk, (size_t)nblk * 2 * sizeof(long long)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL((loop_kernel<NM, NE>), dim3(nblk), dim3(64), 0, 0, out, clk, iters, 0.37f);
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL((loop_kernel<NM, NE>), dim3(nblk), dim3(64), 0, 0, out, clk, iters, 0.37f);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipDeviceSynchronize());
  float ms;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  long long* h = (long long*)malloc((size_t)nblk * 2 * sizeof(long long));
  CHECK(hipMemcpy(h, clk, (size_t)nblk * 2 * sizeof(long long), hipMemcpyDeviceToHost));
  double t = 0, r = 0;
  for (int i = 0; i < nblk; ++i) { t += (double)h[2 * i]; r += (double)h[2 * i + 1]; }
  t /= nblk;
  r /= nblk;
  const double ghz = t / r * 0.1;
  const double tflops = 32768.0 * NM * (double)iters * nblk / (ms * 1e-3) / 1e12;
  printf("| %-24s | %d | %8.1f | %5.2f | %7.0f |\n", name, waves_per_simd, t / iters, ghz, tflops);
  free(h);
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

int main() {
  printf("| loop body per wave | waves/SIMD | clocks per iteration | clock GHz | MFMA TFLOP/s |\n");
  printf("|---|---:|---:|---:|---:|\n");
  for (int w : {1, 2, 4}) {
    run<8, 0>("8 MFMA", w);
    run<0, 32>("32 (exp2, mul)", w);
    run<8, 32>("8 MFMA + 32 (exp2, mul)", w);
    run<16, 32>("16 MFMA + 32 (exp2, mul)", w);
  }
  return 0;
}
