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
  int32_t n_qtiles;     // padded: query tiles per sequence; packed: tile slots
  int32_t n_work;       // total workgroups launched
};

int launch_rel_bucket(int32_t* rel_idx, int32_t max_len, int32_t position_buckets,
                      int32_t max_relative_positions, hipStream_t stream);

// varlen = false: padded layout; true: packed layout.
int launch_fwd(FwdParams& p, int dtype, int d, bool varlen, hipStream_t stream);

}  // namespace dattn

#endif  // DATTN_INTERNAL_H
