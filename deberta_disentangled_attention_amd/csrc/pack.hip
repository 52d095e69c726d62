// Padded <-> packed conversion around the disentangled-attention forward.
//
// The packed layout is the FlashAttention-style one of DisentangledFlash's
// packed unpadded inference (README, "Packed unpadded inference"): the valid
// token rows of a padded batch, concatenated in order, described by int32
// cumulative lengths. The metadata is built once per batch and reused by
// every layer; outputs go back to the padded layout with zero rows where
// the mask is zero.
//
// Metadata, for a [B, L] mask (nonzero = valid):
//   cu[b+1] - cu[b]   = number of valid tokens in row b, cu[0] = 0
//   token_rows[r]     = padded row b*L + l of the r-th valid token in
//                       row-major order, -1 for r >= cu[B]
//   row_to_packed[i]  = r with token_rows[r] = i, or -1
// built in one workgroup for batches up to 4096 rows and 2^18 tokens
// (pack_index_small_kernel), otherwise by three launches:
//   pack_rank_kernel  one workgroup per row: each valid token's rank among
//                     the row's valid tokens (a prefix count of the mask by
//                     wave ballots), and the row's count
//   pack_scan_kernel  one workgroup: running sum of the counts into cu, and
//                     the longest row
//   pack_place_kernel one thread per padded row: its packed index
//                     cu[b] + rank, and the inverse map
// Moving rows is a gather in both directions: one wave per destination row,
// 16 bytes per lane per access, four accesses in flight per lane on wide
// rows. The destination is written in order, so stores stream.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dattn_internal.h"

namespace dattn {

namespace {

constexpr int RANK_THREADS = 256;
constexpr int SCAN_THREADS = 1024;
constexpr int GATHER_THREADS = 256;

__global__ __launch_bounds__(RANK_THREADS) void pack_rank_kernel(
    const uint8_t* __restrict__ mask, int32_t L, int32_t* __restrict__ cu,
    int32_t* __restrict__ row_to_packed) {
  __shared__ int wave_cnt[RANK_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * L;
  const uint64_t below_me = (1ull << lane) - 1ull;
  int base = 0;
  for (int l0 = 0; l0 < L; l0 += RANK_THREADS) {
    const int l = l0 + tid;
    const bool in = l < L;
    const bool valid = in && (mask == nullptr || mask[row0 + l] != 0);
    const uint64_t bal = __ballot(valid);
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int before = base, chunk = 0;
#pragma unroll
    for (int w = 0; w < RANK_THREADS / 64; ++w) {
      before += w < wave ? wave_cnt[w] : 0;
      chunk += wave_cnt[w];
    }
    if (in) row_to_packed[row0 + l] = valid ? before + __popcll(bal & below_me) : -1;
    base += chunk;
    __syncthreads();  // wave_cnt is rewritten by the next chunk
  }
  if (tid == 0) cu[blockIdx.x + 1] = base;
}

// cu[1..B] holds the counts on entry and the inclusive running sums on exit.
__global__ __launch_bounds__(SCAN_THREADS) void pack_scan_kernel(
    int32_t B, int32_t* __restrict__ cu, int32_t* __restrict__ max_len) {
  __shared__ int wave_sum[SCAN_THREADS / 64];
  __shared__ int wave_max[SCAN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0, longest = 0;
  for (int b0 = 0; b0 < B; b0 += SCAN_THREADS) {
    const int b = b0 + tid;
    const int c = b < B ? cu[b + 1] : 0;
    int x = c, m = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      x += lane >= o ? y : 0;
      m = max(m, __shfl_xor(m, o));
    }
    if (lane == 63) wave_sum[wave] = x;
    if (lane == 0) wave_max[wave] = m;
    __syncthreads();
    int before = carry, chunk = 0, cm = 0;
#pragma unroll
    for (int w = 0; w < SCAN_THREADS / 64; ++w) {
      before += w < wave ? wave_sum[w] : 0;
      chunk += wave_sum[w];
      cm = max(cm, wave_max[w]);
    }
    if (b < B) cu[b + 1] = before + x;
    carry += chunk;
    longest = max(longest, cm);
    __syncthreads();
  }
  if (tid == 0) {
    cu[0] = 0;
    if (max_len) *max_len = longest;
  }
}

__global__ void pack_place_kernel(int32_t B, int32_t L, int64_t n, const int32_t* __restrict__ cu,
                                  int32_t* __restrict__ token_rows,
                                  int32_t* __restrict__ row_to_packed) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int rank = row_to_packed[i];
  if (rank >= 0) {
    const int p = cu[i / L] + rank;
    row_to_packed[i] = p;
    token_rows[p] = (int32_t)i;
  }
  // entries at or beyond the packed total are not targets of the scatter
  if (i >= cu[B]) token_rows[i] = -1;
}

// The whole index in one workgroup, for small batches (one launch instead of
// three): wave w counts rows w, w + 16, ...; the counts are scanned in LDS;
// the waves then revisit their rows to place every token.
constexpr int SMALL_THREADS = 1024;
constexpr int SMALL_MAX_ROWS = 4096;
constexpr int64_t SMALL_MAX_TOKENS = 1 << 18;

__global__ __launch_bounds__(SMALL_THREADS) void pack_index_small_kernel(
    const uint8_t* __restrict__ mask, int32_t B, int32_t L, int32_t* __restrict__ cu,
    int32_t* __restrict__ token_rows, int32_t* __restrict__ row_to_packed,
    int32_t* __restrict__ max_len) {
  __shared__ int start[SMALL_MAX_ROWS + 1];
  __shared__ int wave_sum[SMALL_THREADS / 64];
  __shared__ int wave_max[SMALL_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NWAVE = SMALL_THREADS / 64;
  const uint64_t below_me = (1ull << lane) - 1ull;
  auto valid_at = [&](int64_t row0, int l) {
    return l < L && (mask == nullptr || mask[row0 + l] != 0);
  };
  // counts of the rows
  for (int b = wave; b < B; b += NWAVE) {
    const int64_t row0 = (int64_t)b * L;
    int n = 0;
    for (int l0 = 0; l0 < L; l0 += 64) n += __popcll(__ballot(valid_at(row0, l0 + lane)));
    if (lane == 0) start[b + 1] = n;
  }
  __syncthreads();
  // running sums (one chunk of SMALL_THREADS rows at a time) and the maximum
  int carry = 0, longest = 0;
  for (int b0 = 0; b0 < B; b0 += SMALL_THREADS) {
    const int b = b0 + tid;
    const int c = b < B ? start[b + 1] : 0;
    int x = c, m = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      x += lane >= o ? y : 0;
      m = max(m, __shfl_xor(m, o));
    }
    if (lane == 63) wave_sum[wave] = x;
    if (lane == 0) wave_max[wave] = m;
    __syncthreads();
    int before = carry, chunk = 0, cm = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      before += w < wave ? wave_sum[w] : 0;
      chunk += wave_sum[w];
      cm = max(cm, wave_max[w]);
    }
    __syncthreads();   // every count of this chunk is read before it is overwritten
    if (b < B) start[b + 1] = before + x;
    carry += chunk;
    longest = max(longest, cm);
  }
  if (tid == 0) start[0] = 0;
  __syncthreads();
  for (int b = tid; b <= B; b += SMALL_THREADS) cu[b] = start[b];
  if (tid == 0 && max_len) *max_len = longest;
  // place the tokens
  for (int b = wave; b < B; b += NWAVE) {
    const int64_t row0 = (int64_t)b * L;
    int r = start[b];
    for (int l0 = 0; l0 < L; l0 += 64) {
      const int l = l0 + lane;
      const bool valid = valid_at(row0, l);
      const uint64_t bal = __ballot(valid);
      const int p = r + __popcll(bal & below_me);
      if (l < L) row_to_packed[row0 + l] = valid ? p : -1;
      if (valid) token_rows[p] = (int32_t)(row0 + l);
      r += __popcll(bal);
    }
  }
  // entries at or beyond the packed total
  const int64_t n = (int64_t)B * L;
  for (int64_t i = start[B] + tid; i < n; i += SMALL_THREADS) token_rows[i] = -1;
}

// dst row r <- src row idx[r]; an index outside [0, n_src) leaves the row
// untouched (ZERO = false) or writes zeros (ZERO = true).
template <bool ZERO>
__global__ __launch_bounds__(GATHER_THREADS) void gather_rows_kernel(
    const unsigned char* __restrict__ src, int64_t ld_src, int64_t n_src,
    const int32_t* __restrict__ idx, int64_t n_rows, int32_t chunks,
    unsigned char* __restrict__ dst, int64_t ld_dst) {
  const int lane = threadIdx.x & 63;
  const int64_t first = ((int64_t)blockIdx.x * GATHER_THREADS + threadIdx.x) >> 6;
  const int64_t stride = ((int64_t)gridDim.x * GATHER_THREADS) >> 6;
  for (int64_t r = first; r < n_rows; r += stride) {
    const int32_t s = idx[r];
    const bool have = s >= 0 && s < n_src;
    if (!ZERO && !have) continue;
    uint4* d = reinterpret_cast<uint4*>(dst + r * ld_dst);
    if (!have) {
      for (int c = lane; c < chunks; c += 64) d[c] = make_uint4(0u, 0u, 0u, 0u);
      continue;
    }
    const uint4* sp = reinterpret_cast<const uint4*>(src + (int64_t)s * ld_src);
    int c = lane;
    for (; c + 192 < chunks; c += 256) {
      const uint4 a0 = sp[c], a1 = sp[c + 64], a2 = sp[c + 128], a3 = sp[c + 192];
      d[c] = a0;
      d[c + 64] = a1;
      d[c + 128] = a2;
      d[c + 192] = a3;
    }
    for (; c < chunks; c += 64) d[c] = sp[c];
  }
}

}  // namespace

int launch_pack_index(const uint8_t* mask, int32_t B, int32_t L, int32_t* cu,
                      int32_t* token_rows, int32_t* row_to_packed, int32_t* max_len,
                      hipStream_t stream) {
  if (B <= SMALL_MAX_ROWS && (int64_t)B * L <= SMALL_MAX_TOKENS) {
    hipLaunchKernelGGL(pack_index_small_kernel, dim3(1), dim3(SMALL_THREADS), 0, stream, mask, B,
                       L, cu, token_rows, row_to_packed, max_len);
    return hipGetLastError() == hipSuccess ? 0 : 3;
  }
  if (B > 0)
    hipLaunchKernelGGL(pack_rank_kernel, dim3(B), dim3(RANK_THREADS), 0, stream, mask, L, cu,
                       row_to_packed);
  hipLaunchKernelGGL(pack_scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, stream, B, cu, max_len);
  const int64_t n = (int64_t)B * L;
  if (n > 0)
    hipLaunchKernelGGL(pack_place_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, B, L, n, (const int32_t*)cu, token_rows, row_to_packed);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int launch_gather_rows(const void* src, int64_t ld_src, int64_t n_src, const int32_t* idx,
                       int64_t n_rows, int64_t row_bytes, void* dst, int64_t ld_dst,
                       bool zero_missing, hipStream_t stream) {
  const int64_t waves_needed = n_rows;
  const int64_t blocks_needed = (waves_needed + GATHER_THREADS / 64 - 1) / (GATHER_THREADS / 64);
  const unsigned blocks = (unsigned)(blocks_needed < 8192 ? blocks_needed : 8192);
  const int32_t chunks = (int32_t)(row_bytes / 16);
  const unsigned char* s = static_cast<const unsigned char*>(src);
  unsigned char* d = static_cast<unsigned char*>(dst);
  if (zero_missing)
    hipLaunchKernelGGL(gather_rows_kernel<true>, dim3(blocks), dim3(GATHER_THREADS), 0, stream,
                       s, ld_src, n_src, idx, n_rows, chunks, d, ld_dst);
  else
    hipLaunchKernelGGL(gather_rows_kernel<false>, dim3(blocks), dim3(GATHER_THREADS), 0, stream,
                       s, ld_src, n_src, idx, n_rows, chunks, d, ld_dst);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace dattn
