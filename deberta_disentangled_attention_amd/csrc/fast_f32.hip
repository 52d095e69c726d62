// Fast fp32 mode of the forward: fp32 operands in and out, products on the
// fp16 MFMA.
//
// The DisentangledFlash README ("Status") lists an optional fast FP32/TF32
// mode next to strict fp32. CDNA4 has no TF32 matrix instruction; its fp16
// MFMA takes operands with TF32's 10-bit mantissa and accumulates in fp32.
// So the mode rounds q, k, v, qr and kr once to fp16 (round to nearest
// even) into the caller's workspace, runs the fp16 forward on them, and
// widens its output back to fp32. The exponent range is fp16's: inputs
// beyond 65504 in magnitude become infinite, below 2^-24 zero.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dattn_internal.h"

namespace dattn {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void to_f16_kernel(F16Segs segs) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int s = 0; s < segs.n; ++s) {
    const F16Seg g = segs.seg[s];
    const int64_t upr = g.cols / 4;   // 4-element units per row
    const int64_t units = g.rows * upr;
    for (int64_t x = (int64_t)blockIdx.x * kThreads + threadIdx.x; x < units; x += stride) {
      const int64_t r = x / upr, u = x - r * upr;
      const float4 v = *reinterpret_cast<const float4*>(g.src + r * g.ld_src + 4 * u);
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      const h4 h = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
      *reinterpret_cast<h4*>(g.dst + r * g.cols + 4 * u) = h;
    }
  }
}

__global__ __launch_bounds__(kThreads) void to_f32_kernel(const _Float16* __restrict__ src,
                                                          float* __restrict__ dst, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  for (int64_t x = (int64_t)blockIdx.x * kThreads + threadIdx.x; x < n4; x += stride) {
    const h4 h = reinterpret_cast<const h4*>(src)[x];
    reinterpret_cast<float4*>(dst)[x] = make_float4((float)h.x, (float)h.y, (float)h.z, (float)h.w);
  }
}

int grid_for(int64_t units) {
  const int64_t b = (units + kThreads - 1) / kThreads;
  return (int)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

}  // namespace

int launch_to_f16(const F16Segs& segs, hipStream_t stream) {
  int64_t units = 0;
  for (int s = 0; s < segs.n; ++s) units += segs.seg[s].rows * (segs.seg[s].cols / 4);
  if (units == 0) return 0;
  hipLaunchKernelGGL(to_f16_kernel, dim3(grid_for(units)), dim3(kThreads), 0, stream, segs);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int launch_to_f32(const void* src, float* dst, int64_t n, hipStream_t stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(to_f32_kernel, dim3(grid_for(n / 4)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const _Float16*>(src), dst, n / 4);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace dattn
