// Relative-row table for the disentangled-attention forward.
//
// One thread per signed distance r writes clamp(b(r) + s, 0, 2s - 1), the
// row of qr / kr that a pair at distance r reads. b is the DeBERTa-v2 log
// bucket (identity inside |r| <= mid, logarithmic beyond); the pages name the
// method (DisentangledFlash README, "Status") but print no formula, so the
// mapping is the DeBERTa-v2/v3 one its "Attribution" section refers to.
//
// The ceiling must be that of the real number. The argument
//   x = (mid-1) ln(|r|/mid) / ln((M-1)/mid)
// is evaluated in float64; when it lies within 1e-9 of an integer n the
// kernel asks exactly whether x == n, i.e. whether
//   |r|^(mid-1) * mid^n == (M-1)^n * mid^(mid-1),
// by comparing both sides modulo three primes near 2^31. Equality gives
// ceil(x) = n. Otherwise the float64 side of n is used, which is reliable
// unless the argument comes within about 1e-12 of an integer it does not
// reach; no such distance occurs for the parameter sets the tests sweep.
// The forward kernel never evaluates a logarithm: it reads this table.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dattn_internal.h"

namespace dattn {

__device__ __forceinline__ uint32_t mulmod(uint32_t a, uint32_t b, uint32_t p) {
  return (uint32_t)(((uint64_t)a * (uint64_t)b) % p);
}

__device__ uint32_t powmod(uint32_t base, uint32_t e, uint32_t p) {
  uint32_t acc = 1u % p;
  uint32_t x = base % p;
  while (e) {
    if (e & 1u) acc = mulmod(acc, x, p);
    x = mulmod(x, x, p);
    e >>= 1;
  }
  return acc;
}

// true when a^(mid-1) * mid^n == (M-1)^n * mid^(mid-1) modulo three primes
__device__ bool exact_hit(uint32_t a, uint32_t mid, uint32_t Mm1, uint32_t n) {
  const uint32_t primes[3] = {2147483647u, 2147483629u, 2147483587u};
  for (int t = 0; t < 3; ++t) {
    const uint32_t p = primes[t];
    uint32_t lhs = mulmod(powmod(a, mid - 1, p), powmod(mid, n, p), p);
    uint32_t rhs = mulmod(powmod(Mm1, n, p), powmod(mid, mid - 1, p), p);
    if (lhs != rhs) return false;
  }
  return true;
}

// ceil((mid-1) ln(a/mid) / ln((M-1)/mid)) for a > mid
__device__ int log_offset(int a, int mid, int M) {
  if (mid <= 1) return 0;
  if (a == M - 1) return mid - 1;  // the argument is exactly mid - 1 there
  const double x = (double)(mid - 1) * log((double)a / (double)mid) /
                   log((double)(M - 1) / (double)mid);
  const double n = rint(x);
  if (fabs(x - n) <= 1e-9 * fmax(1.0, fabs(x))) {
    if (n >= 0.0 && exact_hit((uint32_t)a, (uint32_t)mid, (uint32_t)(M - 1), (uint32_t)n))
      return (int)n;
  }
  return (int)ceil(x);
}

__global__ void rel_bucket_kernel(int32_t* __restrict__ out, int32_t max_len,
                                  int32_t P, int32_t M) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = 2 * max_len - 1;
  if (idx >= n) return;
  const int r = idx - (max_len - 1);
  int s, b;
  if (P <= 0) {
    s = M;
    b = r;
  } else {
    s = P;
    const int mid = P / 2;
    const int a = r < 0 ? -r : r;
    if (a <= mid) {
      b = r;
    } else {
      const int k = mid + log_offset(a, mid, M);
      b = r > 0 ? k : -k;
    }
  }
  int t = b + s;
  t = t < 0 ? 0 : (t > 2 * s - 1 ? 2 * s - 1 : t);
  out[idx] = t;
}

int launch_rel_bucket(int32_t* rel_idx, int32_t max_len, int32_t P, int32_t M,
                      hipStream_t stream) {
  const int n = 2 * max_len - 1;
  const int threads = 256;
  const int blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(rel_bucket_kernel, dim3(blocks), dim3(threads), 0, stream,
                     rel_idx, max_len, P, M);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace dattn
