// Relative-row table for the disentangled-attention forward.
//
// One thread per signed distance r writes clamp(b(r) + s, 0, 2s - 1), the
// row of qr / kr that a pair at distance r reads. b is the DeBERTa-v2 log
// bucket (identity inside |r| <= mid, logarithmic beyond); the pages name the
// method (DisentangledFlash README, "Status") but print no formula, so the
// mapping is the DeBERTa-v2/v3 one its "Attribution" section refers to.
//
// The ceiling is that of the real number
//   x = e ln(a/mid) / ln((M-1)/mid),   a = |r| > mid, e = mid - 1,
// decided exactly. The kernel evaluates x in float64 as
// e log1p((a-mid)/mid) / log1p((M-1-mid)/mid): every step is within a few
// ulps, so the computed x is within 1e-10 of the real one for every
// supported parameter set (position_buckets <= 4096; only x <= e + 2 < 2^11
// + 2 matters, since every ceiling from e + 2 on gives the table's first or
// last row whatever the parity of P). Where it is more than 1e-9 from an
// integer, its ceiling is the real one. The few distances where it comes
// within 1e-9 of an integer n are found on the host beforehand -- the only
// candidates are a = round(mid ((M-1)/mid)^(n/e)), one per n <= e + 1 -- and decided
// there by comparing (M-1)^n mid^e with a^e mid^n in exact multi-word
// integers (x <= n exactly when the first is not smaller). Those decisions
// reach the kernel as a short list of (a, ceiling) pairs in its arguments.
// At a = M - 1 the argument is exactly e. The forward kernel never evaluates
// a logarithm: it reads this table.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <vector>

#include "dattn_internal.h"

namespace dattn {

constexpr int kMaxFixes = 32;
constexpr double kDeviceBand = 1e-9;   // |x - n| at or below this is settled on the host
constexpr double kHostBand = 1e-8;     // wider, so it covers every device-side candidate

// ceilings decided exactly on the host for distances where float64 is too close to call
struct BucketFixes {
  int32_t count;
  int32_t a[kMaxFixes];
  int32_t k[kMaxFixes];
};

// min(ceil(e ln(a/mid) / ln((M-1)/mid)), e + 2) for a > mid: with either
// parity of P every offset from e + 2 on gives the table's first or last row
__host__ __device__ int log_offset(int a, int mid, int M, const BucketFixes& fx) {
  const int e = mid - 1;
  if (e <= 0) return 0;
  if (a == M - 1) return e;   // the argument is exactly e there
  const double x = (double)e * log1p((double)(a - mid) / (double)mid) /
                   log1p((double)(M - 1 - mid) / (double)mid);
  if (x > (double)(e + 2)) return e + 2;
  const double n = rint(x);
  if (fabs(x - n) <= kDeviceBand) {
    for (int t = 0; t < fx.count; ++t)
      if (fx.a[t] == a) return fx.k[t];
  }
  return (int)ceil(x);
}

// the table entry of distance r
__host__ __device__ int table_entry(int r, int32_t P, int32_t M, const BucketFixes& fx) {
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
      const int k = mid + log_offset(a, mid, M, fx);
      b = r > 0 ? k : -k;
    }
  }
  int t = b + s;
  return t < 0 ? 0 : (t > 2 * s - 1 ? 2 * s - 1 : t);
}

__global__ void rel_bucket_kernel(int32_t* __restrict__ out, int32_t max_len,
                                  int32_t P, int32_t M, BucketFixes fx) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = 2 * max_len - 1;
  if (idx >= n) return;
  out[idx] = table_entry(idx - (max_len - 1), P, M, fx);
}

// ---------------------------------------------------------------------------
// host: exact decisions for the near-integer distances
// ---------------------------------------------------------------------------

namespace {

// little-endian multi-word unsigned integer
typedef std::vector<uint32_t> Big;

void mul_small(Big& x, uint32_t m) {
  uint64_t carry = 0;
  for (uint32_t& w : x) {
    const uint64_t t = (uint64_t)w * m + carry;
    w = (uint32_t)t;
    carry = t >> 32;
  }
  if (carry) x.push_back((uint32_t)carry);
}

// x *= base^n, several factors per pass while their product fits in 32 bits
void mul_pow(Big& x, uint32_t base, int64_t n) {
  if (base == 1) return;
  uint32_t chunk = base;
  int per = 1;
  while ((uint64_t)chunk * base <= 0xffffffffull) { chunk *= base; ++per; }
  for (; n >= per; n -= per) mul_small(x, chunk);
  for (; n > 0; --n) mul_small(x, base);
}

int cmp(const Big& a, const Big& b) {
  if (a.size() != b.size()) return a.size() < b.size() ? -1 : 1;
  for (size_t i = a.size(); i-- > 0;)
    if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
  return 0;
}

// x <= n exactly, i.e. (M-1)^n mid^e >= a^e mid^n
bool arg_at_most(int64_t a, int64_t mid, int64_t Mm1, int64_t e, int64_t n) {
  Big lhs(1, 1u), rhs(1, 1u);
  mul_pow(lhs, (uint32_t)Mm1, n);
  mul_pow(lhs, (uint32_t)mid, e);
  mul_pow(rhs, (uint32_t)a, e);
  mul_pow(rhs, (uint32_t)mid, n);
  return cmp(lhs, rhs) >= 0;
}

// the distances whose float64 argument may fall within the device band of an
// integer, each with its exact ceiling; false when there are too many
bool find_fixes(int32_t max_len, int32_t P, int32_t M, BucketFixes& fx) {
  fx.count = 0;
  if (P <= 0) return true;
  const int64_t mid = P / 2, e = mid - 1, Mm1 = (int64_t)M - 1;
  if (e <= 0) return true;
  const double c = log1p((double)(Mm1 - mid) / (double)mid);
  for (int64_t n = 0; n <= e + 1; ++n) {   // ceilings up to e + 2 matter
    // the argument equals n at a_n = mid ((M-1)/mid)^(n/e); within the host
    // band only round(a_n) can lie (|a - a_n| <= 1e-8 a_n c / e < 0.02)
    const double an = (double)mid * exp((double)n * c / (double)e);
    if (!(an < 2.0 * max_len)) break;   // increasing in n
    const int64_t a = llround(an);
    if (a <= mid || a == Mm1 || a > (int64_t)max_len - 1) continue;
    const double x = (double)e * log1p((double)(a - mid) / (double)mid) / c;
    if (fabs(x - (double)n) > kHostBand) continue;
    if (fx.count == kMaxFixes) return false;
    fx.a[fx.count] = (int32_t)a;
    fx.k[fx.count] = arg_at_most(a, mid, Mm1, e, n) ? (int32_t)n : (int32_t)(n + 1);
    ++fx.count;
  }
  return true;
}

}  // namespace

int32_t rel_bucket_band_host(int32_t max_len, int32_t P, int32_t M) {
  BucketFixes fx;
  if (!find_fixes(max_len, P, M, fx)) return -1;
  const int hi = table_entry(max_len - 1, P, M, fx), lo = table_entry(-(max_len - 1), P, M, fx);
  // the table is non-decreasing: scan down from the longest distance to the
  // first one whose entry (or its mirror's) differs from the end entries
  for (int r = max_len - 1; r >= 1; --r)
    if (table_entry(r, P, M, fx) != hi || table_entry(-r, P, M, fx) != lo) return r + 1;
  return 1;
}

int launch_rel_bucket(int32_t* rel_idx, int32_t max_len, int32_t P, int32_t M,
                      hipStream_t stream) {
  const int n = 2 * max_len - 1;
  const int threads = 256;
  const int blocks = (n + threads - 1) / threads;
  BucketFixes fx;
  if (!find_fixes(max_len, P, M, fx)) return 2;
  hipLaunchKernelGGL(rel_bucket_kernel, dim3(blocks), dim3(threads), 0, stream,
                     rel_idx, max_len, P, M, fx);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace dattn
