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

// Arguments of the backward launches (device pointers; strides in elements).
struct BwdParams {
  const void* q; const void* k; const void* v; const void* o; const void* dout;
  int64_t ld_q, ld_k, ld_v, ld_o, ld_do;
  const float* lse;                 // [tokens, H]
  const void* qr; const void* kr; int64_t ld_rel; int32_t n_rel;
  const int32_t* rel_idx; int32_t rel_max_len;
  const uint8_t* mask; int32_t B, L;         // padded layout
  const int32_t* cu_seqlens; int32_t nseq;   // packed layout
  int64_t tokens;                   // rows of every token array
  int32_t units;                    // sequences
  int32_t H;
  uint32_t flags;
  float tau;
  int32_t band;                     // distances |u| < band are stored by distance
  void* dq; void* dk; void* dv;     // [tokens, H*d]
  void* dqr; void* dkr;             // [n_rel, H*d]
  // workspace
  float* dsum;                      // [tokens, H]
  float* dq_part;                   // [tokens, H, d]
  float* dk_part;                   // [tokens, H, d]
  float* afar;                      // [tokens, H, 2]: query-side sums, u >= band / u <= -band
  float* bfar;                      // [tokens, H, 2]: key-side sums, u >= band / u <= -band
  // dS of the pairs closer than the band by distance u (query minus key),
  // element type, tiled by 32-token groups: [H][groups][dg_rows][32], the
  // entry of token t at distance u in row u + dg_rb of group t / 32
  void* dgq;                        // token t the query: pair (t, t - u)
  void* dgk;                        // token t the key: pair (t + u, t)
  int64_t dg_groups;                // ceil(tokens / 32)
  int32_t dg_rows;                  // rows per group: >= dg_rb + band, even
  int32_t dg_rb;                    // odd, >= band - 1: the row pairs a wave writes start on 128-byte lines
  float* wq;                        // [H, units, 2 band + 1, d]: distance sums with q, then the two far sums
  float* wk;                        // [H, units, 2 band + 1, d]: with k
  int32_t n_qtiles;                 // work items per (unit, head) or tile slots (packed)
  int32_t n_work;
};

// bytes of the backward's workspace, and its layout
int64_t bwd_workspace_bytes(int64_t tokens, int32_t units, int32_t H, int32_t d, int esize,
                            int32_t band);
void bwd_carve_workspace(BwdParams& p, void* ws, int d, int esize);
// the backward's launches on `stream` (p without its workspace pointers carved)
int launch_bwd(BwdParams& p, int dtype, int d, bool varlen, hipStream_t stream);

int launch_rel_bucket(int32_t* rel_idx, int32_t max_len, int32_t position_buckets,
                      int32_t max_relative_positions, hipStream_t stream);
// the table's band: the least W >= 1 such that every entry at distance
// >= W equals the last entry and every entry at distance <= -W the first;
// -1 when the parameters are invalid
int32_t rel_bucket_band_host(int32_t max_len, int32_t P, int32_t M);

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

// fp32 rows (first `cols` of each, row stride ld_src elements) -> contiguous
// fp16 rows; cols a multiple of 4, sources 16-byte aligned
struct F16Seg {
  const float* src;
  int64_t ld_src;
  _Float16* dst;
  int64_t rows, cols;
};
struct F16Segs {
  F16Seg seg[5];
  int n;
};
int launch_to_f16(const F16Segs& segs, hipStream_t stream);
// n fp16 values (n a multiple of 4) -> fp32
int launch_to_f32(const void* src, float* dst, int64_t n, hipStream_t stream);

// qr = E Wq^T + bq, kr = E Wk^T + bk (biases may be null); strides in elements
int launch_rel_proj(const void* E, int64_t ld_e, const void* Wq, const void* Wk, int64_t ld_w,
                    const void* bq, const void* bk, void* qr, void* kr, int64_t ld_out,
                    int32_t n_rel, int32_t hidden, int32_t HD, int dtype, hipStream_t stream);

}  // namespace dattn

#endif  // DATTN_INTERNAL_H
