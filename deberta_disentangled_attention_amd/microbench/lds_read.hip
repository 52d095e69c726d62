// LDS read throughput of gfx950 for the two operand reads of the forward's
// far-tile loop: ds_read_b128 (K operand) and the transposing
// ds_read_b64_tr_b16 (V^T operand), alone and with 32x32x16 bf16 MFMAs
// issued by the same waves. Workgroups of 4 waves, 1 or 2 per CU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)

// TR: 0 ds_read_b128 (16 bytes per lane), 1 ds_read_b64_tr_b16 (8 bytes)
template <int TR, int NMF>
__global__ __launch_bounds__(256) void lds_kernel(uint32_t* out, int iters, float seed) {
  __shared__ __attribute__((aligned(16))) unsigned char sm[32768];
  for (int x = threadIdx.x; x < 32768 / 16; x += 256)
    reinterpret_cast<uint4*>(sm)[x] = make_uint4(x, x + 1, x + 2, x + 3);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint4 accv = make_uint4(0, 0, 0, 0);
  f32x16 acc[4] = {};
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (lane + i));
    b[i] = (__bf16)(seed + i);
  }
  for (int it = 0; it < iters; ++it) {
    // eight reads of 1 KB (b128) or 512 B (tr_b16) per wave, inside 16 KB
    const int base = ((it * 1024) + wave * 4096) & 16383;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (TR == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(sm + base + k * 1024 + lane * 16);
        accv.x ^= v.x; accv.y ^= v.y; accv.z ^= v.z; accv.w ^= v.w;
      } else {
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(sm + base + k * 1024 + lane * 8));
        const uint2 u = __builtin_bit_cast(uint2, v);
        accv.x ^= u.x; accv.y ^= u.y;
      }
    }
#pragma unroll
    for (int m = 0; m < NMF; ++m) acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
  }
  float s = 0.f;
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 16; ++r) s += acc[m][r];
  out[blockIdx.x * 256 + threadIdx.x] = accv.x ^ accv.y ^ accv.z ^ accv.w ^ (uint32_t)s;
}

template <int TR, int NMF>
void run(const char* name, int wg_per_cu) {
  const int nblk = 256 * wg_per_cu, iters = 4000;
  uint32_t* out;
  CHECK(hipMalloc(&out, (size_t)nblk * 256 * 4));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL((lds_kernel<TR, NMF>), dim3(nblk), dim3(256), 0, 0, out, iters, 0.3f);
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL((lds_kernel<TR, NMF>), dim3(nblk), dim3(256), 0, 0, out, iters, 0.3f);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipDeviceSynchronize());
  float ms;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double bytes = (double)nblk * 4 * iters * 8 * 64 * (TR == 0 ? 16 : 8);
  const double flop = (double)nblk * 4 * iters * NMF * 32768.0;
  printf("| %-18s | %d | %6.1f | %6.0f |\n", name, wg_per_cu, bytes / (ms * 1e-3) / 256 / 1e9, flop / (ms * 1e-3) / 1e12);
  CHECK(hipFree(out));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

int main() {
  printf("| per wave and iteration | WG/CU | LDS GB/s per CU | MFMA TFLOP/s |\n");
  printf("|---|---:|---:|---:|\n");
  for (int w : {1, 2}) {
    run<0, 0>("8 b128", w);
    run<1, 0>("8 tr_b16", w);
    run<0, 8>("8 b128 + 8 MFMA", w);
    run<1, 8>("8 tr_b16 + 8 MFMA", w);
    run<0, 16>("8 b128 + 16 MFMA", w);
  }
  return 0;
}
