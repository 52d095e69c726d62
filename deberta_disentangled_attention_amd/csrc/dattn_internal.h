// Internal interface between the C ABI (dattn_api.hip) and the kernels.
#ifndef DATTN_INTERNAL_H
#define DATTN_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dattn {

// Arguments of one forward launch. Pointers are device pointers; strides
// are in elements.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t ld_q, ld_k, ld_v;
  const void* qr;
  const void* kr;
  int64_t ld_rel;
  int32_t n_rel;
  const int32_t* rel_idx;
  int32_t rel_max_len;
  // padded layout
  const uint8_t* mask;  // [B, L] or null
  int32_t B, L;
  // packed layout
  const int32_t* cu_seqlens;
  int32_t nseq;
  int64_t total_tokens;
  void* out;
  int32_t H;
  uint32_t flags;
  float scale_log2;     // softmax scale times log2(e)
  float* lse;           // [tokens, H] natural log of each row's sum of exp(scores), or null
  int32_t max_seqlen;   // padded: L; packed: the caller's bound on every length
  int32_t n_qtiles;     // padded: query tiles per sequence; packed: tile slots
  int32_t n_work;       // work items (query tiles of every (sequence, head)), one per workgroup
  int32_t qt_major;     // padded only: items ordered query tile first
};

int launch_rel_bucket(int32_t* rel_idx, int32_t max_len, int32_t position_buckets,
                      int32_t max_relative_positions, hipStream_t stream);

// varlen = false: padded layout; true: packed layout.
int launch_fwd(FwdParams& p, int dtype, int d, bool varlen, hipStream_t stream);

// packing metadata of a [B, L] mask (null = all valid); max_len may be null
int launch_pack_index(const uint8_t* mask, int32_t B, int32_t L, int32_t* cu,
                      int32_t* token_rows, int32_t* row_to_packed, int32_t* max_len,
                      hipStream_t stream);

// dst row r <- src row idx[r] for r < n_rows; strides and row_bytes in
// bytes (multiples of 16). Indices outside [0, n_src) skip the row, or zero
// it when zero_missing.
int launch_gather_rows(const void* src, int64_t ld_src, int64_t n_src, const int32_t* idx,
                       int64_t n_rows, int64_t row_bytes, void* dst, int64_t ld_dst,
                       bool zero_missing, hipStream_t stream);

// qr = E Wq^T + bq, kr = E Wk^T + bk (biases may be null); strides in elements
int launch_rel_proj(const void* E, int64_t ld_e, const void* Wq, const void* Wk, int64_t ld_w,
                    const void* bq, const void* bk, void* qr, void* kr, int64_t ld_out,
                    int32_t n_rel, int32_t hidden, int32_t HD, int dtype, hipStream_t stream);

}  // namespace dattn

#endif  // DATTN_INTERNAL_H
