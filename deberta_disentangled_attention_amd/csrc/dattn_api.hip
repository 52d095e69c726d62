// C ABI of libdattn.so: argument validation and dispatch. Every check runs
// on the host before any HIP call, so a rejected call touches no device
// state. There is no fallback path: unsupported cases return a status.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/dattn.h"
#include "dattn_internal.h"

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
// int32 arrays are read and written as whole words
bool aligned4(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3u) == 0; }

int esize_of(int32_t dtype) { return dtype == DATTN_F32 ? 4 : 2; }

// checks shared by both layouts; seq_bound is L (padded) or max_seqlen
int check_common(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                 int64_t ld_v, const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                 const int32_t* rel_idx, int32_t rel_max_len, const void* out, int32_t H,
                 int32_t d, int32_t dtype, uint32_t flags, float scale, int32_t seq_bound) {
  if (!q || !k || !v || !out) return DATTN_ERR_INVALID_ARGUMENT;
  if (H < 1) return DATTN_ERR_INVALID_ARGUMENT;
  if (flags & ~(DATTN_C2P | DATTN_P2C)) return DATTN_ERR_INVALID_ARGUMENT;
  if (isnan(scale)) return DATTN_ERR_INVALID_ARGUMENT;
  if (dtype != DATTN_F32 && dtype != DATTN_F16 && dtype != DATTN_BF16) return DATTN_ERR_UNSUPPORTED;
  if (d != 32 && d != 64 && d != 128) return DATTN_ERR_UNSUPPORTED;
  if (seq_bound > DATTN_MAX_SEQLEN) return DATTN_ERR_UNSUPPORTED;
  const int64_t hd = (int64_t)H * d;
  if (ld_q < hd || ld_k < hd || ld_v < hd) return DATTN_ERR_INVALID_ARGUMENT;
  const int es = esize_of(dtype);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return DATTN_ERR_UNSUPPORTED;
  if ((ld_q * es) % 16 || (ld_k * es) % 16 || (ld_v * es) % 16) return DATTN_ERR_UNSUPPORTED;
  if (flags) {
    if (!qr || !kr || !rel_idx) return DATTN_ERR_INVALID_ARGUMENT;
    if (!aligned4(rel_idx)) return DATTN_ERR_UNSUPPORTED;
    if (n_rel < 1 || ld_rel < hd) return DATTN_ERR_INVALID_ARGUMENT;
    if (rel_max_len < seq_bound || rel_max_len < 1) return DATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(qr) || !aligned16(kr) || (ld_rel * es) % 16) return DATTN_ERR_UNSUPPORTED;
    if ((int64_t)n_rel * ld_rel * es > INT32_MAX) return DATTN_ERR_UNSUPPORTED;  // row offsets are 31-bit
  }
  return DATTN_OK;
}

float scale_log2(int32_t d, uint32_t flags, float scale) {
  const int terms = ((flags & DATTN_C2P) ? 1 : 0) + ((flags & DATTN_P2C) ? 1 : 0);
  const double tau = scale > 0.f ? (double)scale : 1.0 / sqrt((double)d * (1 + terms));
  return (float)(tau * 1.4426950408889634);
}

}  // namespace

extern "C" {

int rel_bucket(int32_t* rel_idx, int32_t max_len, int32_t position_buckets,
               int32_t max_relative_positions, hipStream_t stream) {
  if (!rel_idx || max_len < 1) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(rel_idx)) return DATTN_ERR_UNSUPPORTED;
  if (max_len > 65536) return DATTN_ERR_UNSUPPORTED;
  if (position_buckets > 4096) return DATTN_ERR_UNSUPPORTED;
  if (position_buckets > 0) {
    const int mid = position_buckets / 2;
    if (mid < 1) return DATTN_ERR_INVALID_ARGUMENT;
    if (max_relative_positions - 1 <= mid) return DATTN_ERR_INVALID_ARGUMENT;
  } else if (max_relative_positions < 1) {
    return DATTN_ERR_INVALID_ARGUMENT;
  }
  return dattn::launch_rel_bucket(rel_idx, max_len, position_buckets, max_relative_positions, stream);
}

static int fwd_padded(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                      int64_t ld_v, const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                      const int32_t* rel_idx, int32_t rel_max_len, const uint8_t* mask, void* out,
                      int32_t B, int32_t L, int32_t H, int32_t d, int32_t dtype, uint32_t flags,
                      float scale, float* lse, hipStream_t stream) {
  if (B < 0 || L < 0) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(lse)) return DATTN_ERR_UNSUPPORTED;
  int st = check_common(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len,
                        out, H, d, dtype, flags, scale, L);
  if (st != DATTN_OK) return st;
  if ((int64_t)B * L == 0) return DATTN_OK;
  dattn::FwdParams p = {};
  p.q = q; p.k = k; p.v = v;
  p.ld_q = ld_q; p.ld_k = ld_k; p.ld_v = ld_v;
  p.qr = qr; p.kr = kr; p.ld_rel = ld_rel; p.n_rel = n_rel;
  p.rel_idx = rel_idx; p.rel_max_len = rel_max_len;
  p.mask = mask; p.B = B; p.L = L; p.max_seqlen = L;
  p.cu_seqlens = nullptr; p.nseq = 0; p.total_tokens = (int64_t)B * L;
  p.out = out; p.H = H; p.flags = flags;
  p.scale_log2 = scale_log2(d, flags, scale);
  p.lse = lse;
  return dattn::launch_fwd(p, dtype, d, false, stream);
}

static int fwd_varlen(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                      int64_t ld_v, const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                      const int32_t* rel_idx, int32_t rel_max_len, const int32_t* cu_seqlens,
                      int32_t nseq, int32_t max_seqlen, int64_t total_tokens, void* out, int32_t H,
                      int32_t d, int32_t dtype, uint32_t flags, float scale, float* lse,
                      hipStream_t stream) {
  if (nseq < 0 || total_tokens < 0 || max_seqlen < 0) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(lse)) return DATTN_ERR_UNSUPPORTED;
  if (!cu_seqlens) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(cu_seqlens)) return DATTN_ERR_UNSUPPORTED;
  int st = check_common(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len,
                        out, H, d, dtype, flags, scale, max_seqlen);
  if (st != DATTN_OK) return st;
  if (nseq == 0 || total_tokens == 0) return DATTN_OK;
  dattn::FwdParams p = {};
  p.q = q; p.k = k; p.v = v;
  p.ld_q = ld_q; p.ld_k = ld_k; p.ld_v = ld_v;
  p.qr = qr; p.kr = kr; p.ld_rel = ld_rel; p.n_rel = n_rel;
  p.rel_idx = rel_idx; p.rel_max_len = rel_max_len;
  p.mask = nullptr; p.B = 0; p.L = 0; p.max_seqlen = max_seqlen;
  p.cu_seqlens = cu_seqlens; p.nseq = nseq; p.total_tokens = total_tokens;
  p.out = out; p.H = H; p.flags = flags;
  p.scale_log2 = scale_log2(d, flags, scale);
  p.lse = lse;
  return dattn::launch_fwd(p, dtype, d, true, stream);
}

int dattn_fwd_padded(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                     int64_t ld_v, const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                     const int32_t* rel_idx, int32_t rel_max_len, const uint8_t* mask, void* out,
                     int32_t B, int32_t L, int32_t H, int32_t d, int32_t dtype, uint32_t flags,
                     float scale, hipStream_t stream) {
  return fwd_padded(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len, mask,
                    out, B, L, H, d, dtype, flags, scale, nullptr, stream);
}

int dattn_fwd_padded_lse(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                         int64_t ld_v, const void* qr, const void* kr, int64_t ld_rel,
                         int32_t n_rel, const int32_t* rel_idx, int32_t rel_max_len,
                         const uint8_t* mask, void* out, float* lse, int32_t B, int32_t L,
                         int32_t H, int32_t d, int32_t dtype, uint32_t flags, float scale,
                         hipStream_t stream) {
  if (!lse) return DATTN_ERR_INVALID_ARGUMENT;
  return fwd_padded(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len, mask,
                    out, B, L, H, d, dtype, flags, scale, lse, stream);
}

int dattn_fwd_varlen(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                     int64_t ld_v, const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                     const int32_t* rel_idx, int32_t rel_max_len, const int32_t* cu_seqlens,
                     int32_t nseq, int32_t max_seqlen, int64_t total_tokens, void* out, int32_t H,
                     int32_t d, int32_t dtype, uint32_t flags, float scale, hipStream_t stream) {
  return fwd_varlen(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len,
                    cu_seqlens, nseq, max_seqlen, total_tokens, out, H, d, dtype, flags, scale,
                    nullptr, stream);
}

int dattn_fwd_varlen_lse(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                         int64_t ld_v, const void* qr, const void* kr, int64_t ld_rel,
                         int32_t n_rel, const int32_t* rel_idx, int32_t rel_max_len,
                         const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                         int64_t total_tokens, void* out, float* lse, int32_t H, int32_t d,
                         int32_t dtype, uint32_t flags, float scale, hipStream_t stream) {
  if (!lse) return DATTN_ERR_INVALID_ARGUMENT;
  return fwd_varlen(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len,
                    cu_seqlens, nseq, max_seqlen, total_tokens, out, H, d, dtype, flags, scale,
                    lse, stream);
}

// ---------------------------------------------------------------------------
// fast fp32 forward: operands rounded to fp16 in the workspace, the fp16
// forward, the output widened back to fp32
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

int64_t al256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t fast_ws_bytes(int64_t rows, int32_t n_rel, int32_t H, int32_t d) {
  const int64_t hd = (int64_t)H * d;
  return 4 * al256(rows * hd * 2) + 2 * al256((int64_t)n_rel * hd * 2);
}

// fp16 copies of the operands in the workspace, then the fp16 forward into
// the workspace's output rows, then those rows widened into out
template <class Run>
int fast_f32(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k, int64_t ld_v,
             const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel, uint32_t flags,
             void* out, int64_t rows, int32_t H, int32_t d, void* workspace, int64_t workspace_bytes,
             hipStream_t stream, Run run) {
  if (!workspace) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace)) return DATTN_ERR_UNSUPPORTED;
  if (rows == 0) return DATTN_OK;
  const int32_t nr = flags ? n_rel : 0;
  if (workspace_bytes < fast_ws_bytes(rows, nr, H, d)) return DATTN_ERR_INVALID_ARGUMENT;
  const int64_t hd = (int64_t)H * d;
  unsigned char* w = reinterpret_cast<unsigned char*>(workspace);
  auto take = [&](int64_t n) {
    _Float16* p = reinterpret_cast<_Float16*>(w);
    w += al256(n * 2);
    return p;
  };
  _Float16 *q16 = take(rows * hd), *k16 = take(rows * hd), *v16 = take(rows * hd), *o16 = take(rows * hd);
  _Float16 *qr16 = nullptr, *kr16 = nullptr;
  dattn::F16Segs segs = {};
  segs.seg[0] = {reinterpret_cast<const float*>(q), ld_q, q16, rows, hd};
  segs.seg[1] = {reinterpret_cast<const float*>(k), ld_k, k16, rows, hd};
  segs.seg[2] = {reinterpret_cast<const float*>(v), ld_v, v16, rows, hd};
  segs.n = 3;
  if (nr) {
    qr16 = take((int64_t)nr * hd);
    kr16 = take((int64_t)nr * hd);
    segs.seg[3] = {reinterpret_cast<const float*>(qr), ld_rel, qr16, nr, hd};
    segs.seg[4] = {reinterpret_cast<const float*>(kr), ld_rel, kr16, nr, hd};
    segs.n = 5;
  }
  int st = dattn::launch_to_f16(segs, stream);
  if (st != DATTN_OK) return st;
  st = run(q16, k16, v16, hd, qr16, kr16, o16);
  if (st != DATTN_OK) return st;
  return dattn::launch_to_f32(o16, reinterpret_cast<float*>(out), rows * hd, stream);
}

}  // namespace

extern "C" {

int64_t dattn_fwd_f32fast_workspace_size(int64_t rows, int32_t n_rel, int32_t H, int32_t d) {
  if (rows < 0 || n_rel < 0 || H < 1) return -1;
  if (d != 32 && d != 64 && d != 128) return -1;
  return fast_ws_bytes(rows, n_rel, H, d);
}

int dattn_fwd_padded_f32fast(const void* q, const void* k, const void* v, int64_t ld_q,
                             int64_t ld_k, int64_t ld_v, const void* qr, const void* kr,
                             int64_t ld_rel, int32_t n_rel, const int32_t* rel_idx,
                             int32_t rel_max_len, const uint8_t* mask, void* out, int32_t B,
                             int32_t L, int32_t H, int32_t d, uint32_t flags, float scale,
                             void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || L < 0) return DATTN_ERR_INVALID_ARGUMENT;
  int st = check_common(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len,
                        out, H, d, DATTN_F32, flags, scale, L);
  if (st != DATTN_OK) return st;
  return fast_f32(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, flags, out, (int64_t)B * L, H,
                  d, workspace, workspace_bytes, stream,
                  [&](const void* q16, const void* k16, const void* v16, int64_t hd,
                      const void* qr16, const void* kr16, void* o16) {
                    return fwd_padded(q16, k16, v16, hd, hd, hd, qr16, kr16, hd, n_rel, rel_idx,
                                      rel_max_len, mask, o16, B, L, H, d, DATTN_F16, flags, scale,
                                      nullptr, stream);
                  });
}

int dattn_fwd_varlen_f32fast(const void* q, const void* k, const void* v, int64_t ld_q,
                             int64_t ld_k, int64_t ld_v, const void* qr, const void* kr,
                             int64_t ld_rel, int32_t n_rel, const int32_t* rel_idx,
                             int32_t rel_max_len, const int32_t* cu_seqlens, int32_t nseq,
                             int32_t max_seqlen, int64_t total_tokens, void* out, int32_t H,
                             int32_t d, uint32_t flags, float scale, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream) {
  if (nseq < 0 || total_tokens < 0 || max_seqlen < 0) return DATTN_ERR_INVALID_ARGUMENT;
  if (!cu_seqlens) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(cu_seqlens)) return DATTN_ERR_UNSUPPORTED;
  int st = check_common(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len,
                        out, H, d, DATTN_F32, flags, scale, max_seqlen);
  if (st != DATTN_OK) return st;
  if (nseq == 0) return DATTN_OK;
  return fast_f32(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, flags, out, total_tokens, H, d,
                  workspace, workspace_bytes, stream,
                  [&](const void* q16, const void* k16, const void* v16, int64_t hd,
                      const void* qr16, const void* kr16, void* o16) {
                    return fwd_varlen(q16, k16, v16, hd, hd, hd, qr16, kr16, hd, n_rel, rel_idx,
                                      rel_max_len, cu_seqlens, nseq, max_seqlen, total_tokens, o16,
                                      H, d, DATTN_F16, flags, scale, nullptr, stream);
                  });
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------

int32_t rel_bucket_band(int32_t max_len, int32_t position_buckets, int32_t max_relative_positions) {
  if (max_len < 1 || max_len > 65536) return -1;
  if (position_buckets > 4096) return -1;
  if (position_buckets > 0) {
    const int mid = position_buckets / 2;
    if (mid < 1 || max_relative_positions - 1 <= mid) return -1;
  } else if (max_relative_positions < 1) {
    return -1;
  }
  return dattn::rel_bucket_band_host(max_len, position_buckets, max_relative_positions);
}

int64_t dattn_bwd_workspace_size(int64_t total_tokens, int32_t nseq, int32_t H, int32_t d,
                                 int32_t dtype, int32_t band) {
  if (total_tokens < 0 || nseq < 0 || H < 1 || band < 1) return -1;
  if (d != 32 && d != 64 && d != 128) return -1;
  if (dtype != DATTN_F32 && dtype != DATTN_F16 && dtype != DATTN_BF16) return -1;
  return dattn::bwd_workspace_bytes(total_tokens, nseq, H, d, esize_of(dtype), band);
}

static int bwd_common(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                      int64_t ld_v, const void* out, const void* dout, int64_t ld_o, int64_t ld_do,
                      const float* lse, const void* qr, const void* kr, int64_t ld_rel,
                      int32_t n_rel, const int32_t* rel_idx, int32_t rel_max_len, int32_t band,
                      void* dq, void* dk, void* dv, void* dqr, void* dkr, void* workspace,
                      int64_t workspace_bytes, int32_t H, int32_t d, int32_t dtype, uint32_t flags,
                      float scale, int32_t seq_bound, dattn::BwdParams& p) {
  int st = check_common(q, k, v, ld_q, ld_k, ld_v, qr, kr, ld_rel, n_rel, rel_idx, rel_max_len,
                        dq, H, d, dtype, flags, scale, seq_bound);
  if (st != DATTN_OK) return st;
  if (!out || !dout || !lse || !dk || !dv || !workspace) return DATTN_ERR_INVALID_ARGUMENT;
  const int64_t hd = (int64_t)H * d;
  if (ld_o < hd || ld_do < hd) return DATTN_ERR_INVALID_ARGUMENT;
  const int es = esize_of(dtype);
  if (!aligned16(out) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse) ||
      !aligned16(workspace))
    return DATTN_ERR_UNSUPPORTED;
  if ((ld_o * es) % 16 || (ld_do * es) % 16) return DATTN_ERR_UNSUPPORTED;
  if (flags) {
    if (!dqr || !dkr) return DATTN_ERR_INVALID_ARGUMENT;
    if (!aligned16(dqr) || !aligned16(dkr)) return DATTN_ERR_UNSUPPORTED;
  }
  // the distance store covers |u| < band; the table must be constant beyond
  if (!flags) band = 1;   // ignored: no pair reads a table
  if (band < 1 || band > (flags ? rel_max_len : 1)) return DATTN_ERR_INVALID_ARGUMENT;
  p = dattn::BwdParams{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.dout = dout;
  p.ld_q = ld_q; p.ld_k = ld_k; p.ld_v = ld_v; p.ld_o = ld_o; p.ld_do = ld_do;
  p.lse = lse;
  p.qr = qr; p.kr = kr; p.ld_rel = ld_rel; p.n_rel = n_rel;
  p.rel_idx = rel_idx; p.rel_max_len = rel_max_len;
  p.H = H; p.flags = flags;
  const int terms = ((flags & DATTN_C2P) ? 1 : 0) + ((flags & DATTN_P2C) ? 1 : 0);
  p.tau = scale > 0.f ? scale : (float)(1.0 / sqrt((double)d * (1 + terms)));
  p.band = band;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dqr = dqr; p.dkr = dkr;
  (void)workspace_bytes;
  return DATTN_OK;
}

int dattn_bwd_padded(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                     int64_t ld_v, const void* out, const void* dout, int64_t ld_o, int64_t ld_do,
                     const float* lse, const void* qr, const void* kr, int64_t ld_rel,
                     int32_t n_rel, const int32_t* rel_idx, int32_t rel_max_len, int32_t band,
                     const uint8_t* mask, void* dq, void* dk, void* dv, void* dqr, void* dkr,
                     void* workspace, int64_t workspace_bytes, int32_t B, int32_t L, int32_t H,
                     int32_t d, int32_t dtype, uint32_t flags, float scale, hipStream_t stream) {
  if (B < 0 || L < 0) return DATTN_ERR_INVALID_ARGUMENT;
  dattn::BwdParams p;
  int st = bwd_common(q, k, v, ld_q, ld_k, ld_v, out, dout, ld_o, ld_do, lse, qr, kr, ld_rel, n_rel,
                      rel_idx, rel_max_len, band, dq, dk, dv, dqr, dkr, workspace, workspace_bytes,
                      H, d, dtype, flags, scale, L, p);
  if (st != DATTN_OK) return st;
  if ((int64_t)B * L == 0) return DATTN_OK;
  const int64_t need = dattn::bwd_workspace_bytes((int64_t)B * L, B, H, d, esize_of(dtype), p.band);
  if (workspace_bytes < need) return DATTN_ERR_INVALID_ARGUMENT;
  p.mask = mask; p.B = B; p.L = L;
  p.cu_seqlens = nullptr; p.nseq = 0;
  p.tokens = (int64_t)B * L; p.units = B;
  dattn::bwd_carve_workspace(p, workspace, d, esize_of(dtype));
  return dattn::launch_bwd(p, dtype, d, false, stream);
}

int dattn_bwd_varlen(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                     int64_t ld_v, const void* out, const void* dout, int64_t ld_o, int64_t ld_do,
                     const float* lse, const void* qr, const void* kr, int64_t ld_rel,
                     int32_t n_rel, const int32_t* rel_idx, int32_t rel_max_len, int32_t band,
                     const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                     int64_t total_tokens, void* dq, void* dk, void* dv, void* dqr, void* dkr,
                     void* workspace, int64_t workspace_bytes, int32_t H, int32_t d, int32_t dtype,
                     uint32_t flags, float scale, hipStream_t stream) {
  if (nseq < 0 || total_tokens < 0 || max_seqlen < 0) return DATTN_ERR_INVALID_ARGUMENT;
  if (!cu_seqlens) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(cu_seqlens)) return DATTN_ERR_UNSUPPORTED;
  dattn::BwdParams p;
  int st = bwd_common(q, k, v, ld_q, ld_k, ld_v, out, dout, ld_o, ld_do, lse, qr, kr, ld_rel, n_rel,
                      rel_idx, rel_max_len, band, dq, dk, dv, dqr, dkr, workspace, workspace_bytes,
                      H, d, dtype, flags, scale, max_seqlen, p);
  if (st != DATTN_OK) return st;
  if (nseq == 0 || total_tokens == 0) return DATTN_OK;
  const int64_t need = dattn::bwd_workspace_bytes(total_tokens, nseq, H, d, esize_of(dtype), p.band);
  if (workspace_bytes < need) return DATTN_ERR_INVALID_ARGUMENT;
  p.mask = nullptr; p.B = 0; p.L = 0;
  p.cu_seqlens = cu_seqlens; p.nseq = nseq;
  p.tokens = total_tokens; p.units = nseq;
  dattn::bwd_carve_workspace(p, workspace, d, esize_of(dtype));
  return dattn::launch_bwd(p, dtype, d, true, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// allocation-free backward: the workspace lives in a fixed device array
// ---------------------------------------------------------------------------

// One copy per GPU, held from module load until the process ends. Host code
// never passes `scratch` itself to a kernel (on the host the name is only a
// stand-in): it uses the address hipGetSymbolAddress returns on each device.
static __device__ __align__(256) unsigned char scratch[DATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // scratch's address on each device, once looked up

// address of scratch on the current device (looked up on the first call there)
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DATTN_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DATTN_OK;
}

}  // namespace

extern "C" {

int dattn_bwd_varlen_noalloc(const void* q, const void* k, const void* v, int64_t ld_q,
                             int64_t ld_k, int64_t ld_v, const void* out, const void* dout,
                             int64_t ld_o, int64_t ld_do, const float* lse, const void* qr,
                             const void* kr, int64_t ld_rel, int32_t n_rel, const int32_t* rel_idx,
                             int32_t rel_max_len, int32_t band, const int32_t* cu_seqlens,
                             int32_t nseq, int32_t max_seqlen, int64_t total_tokens, void* dq,
                             void* dk, void* dv, void* dqr, void* dkr, int32_t H, int32_t d,
                             int32_t dtype, uint32_t flags, float scale, hipStream_t stream) {
  if (nseq < 0 || total_tokens < 0 || max_seqlen < 0) return DATTN_ERR_INVALID_ARGUMENT;
  if (!cu_seqlens) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(cu_seqlens)) return DATTN_ERR_UNSUPPORTED;
  dattn::BwdParams p;
  // the checks of dattn_bwd_varlen, with a stand-in workspace pointer
  int st = bwd_common(q, k, v, ld_q, ld_k, ld_v, out, dout, ld_o, ld_do, lse, qr, kr, ld_rel, n_rel,
                      rel_idx, rel_max_len, band, dq, dk, dv, dqr, dkr, reinterpret_cast<void*>(256),
                      0, H, d, dtype, flags, scale, max_seqlen, p);
  if (st != DATTN_OK) return st;
  if (nseq == 0 || total_tokens == 0) return DATTN_OK;
  const int64_t need = dattn::bwd_workspace_bytes(total_tokens, nseq, H, d, esize_of(dtype), p.band);
  if (need > DATTN_NOALLOC_SCRATCH_BYTES) return DATTN_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != DATTN_OK) return st;
  p.mask = nullptr; p.B = 0; p.L = 0;
  p.cu_seqlens = cu_seqlens; p.nseq = nseq;
  p.tokens = total_tokens; p.units = nseq;
  dattn::bwd_carve_workspace(p, ws, d, esize_of(dtype));
  return dattn::launch_bwd(p, dtype, d, true, stream);
}

int dattn_pack_index(const uint8_t* mask, int32_t B, int32_t L, int32_t* cu_seqlens,
                     int32_t* token_rows, int32_t* row_to_packed, int32_t* max_seqlen,
                     hipStream_t stream) {
  if (B < 0 || L < 0 || !cu_seqlens) return DATTN_ERR_INVALID_ARGUMENT;
  const int64_t n = (int64_t)B * L;
  if (n > INT32_MAX || B == INT32_MAX) return DATTN_ERR_UNSUPPORTED;  // int32 indices
  if (n > 0 && (!token_rows || !row_to_packed)) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(cu_seqlens) || !aligned4(token_rows) || !aligned4(row_to_packed) ||
      !aligned4(max_seqlen))
    return DATTN_ERR_UNSUPPORTED;
  return dattn::launch_pack_index(mask, B, L, cu_seqlens, token_rows, row_to_packed, max_seqlen,
                                  stream);
}

static int gather_rows(const void* src, int64_t ld_src_bytes, int64_t n_src, const int32_t* index,
                       int64_t n_rows, int64_t row_bytes, void* dst, int64_t ld_dst_bytes,
                       bool zero_missing, hipStream_t stream) {
  if (n_rows < 0 || n_src < 0 || row_bytes < 0) return DATTN_ERR_INVALID_ARGUMENT;
  if (n_rows == 0 || row_bytes == 0) return DATTN_OK;
  if (!src || !dst || !index) return DATTN_ERR_INVALID_ARGUMENT;
  if (!aligned4(index)) return DATTN_ERR_UNSUPPORTED;
  if (ld_src_bytes < row_bytes || ld_dst_bytes < row_bytes) return DATTN_ERR_INVALID_ARGUMENT;
  if (row_bytes % 16 || ld_src_bytes % 16 || ld_dst_bytes % 16) return DATTN_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst)) return DATTN_ERR_UNSUPPORTED;
  if (row_bytes / 16 > INT32_MAX) return DATTN_ERR_UNSUPPORTED;
  return dattn::launch_gather_rows(src, ld_src_bytes, n_src, index, n_rows, row_bytes, dst,
                                   ld_dst_bytes, zero_missing, stream);
}

int dattn_pack_rows(const void* src, int64_t ld_src_bytes, int64_t n_src,
                    const int32_t* token_rows, int64_t n_rows, int64_t row_bytes, void* dst,
                    int64_t ld_dst_bytes, hipStream_t stream) {
  return gather_rows(src, ld_src_bytes, n_src, token_rows, n_rows, row_bytes, dst, ld_dst_bytes,
                     false, stream);
}

int dattn_unpack_rows(const void* src, int64_t ld_src_bytes, int64_t n_src,
                      const int32_t* row_to_packed, int64_t n_rows, int64_t row_bytes, void* dst,
                      int64_t ld_dst_bytes, hipStream_t stream) {
  return gather_rows(src, ld_src_bytes, n_src, row_to_packed, n_rows, row_bytes, dst,
                     ld_dst_bytes, true, stream);
}

int dattn_rel_proj(const void* E, int64_t ld_e, const void* Wq, const void* Wk, int64_t ld_w,
                   const void* bq, const void* bk, void* qr, void* kr, int64_t ld_out,
                   int32_t n_rel, int32_t hidden, int32_t HD, int32_t dtype, hipStream_t stream) {
  if (n_rel < 0 || hidden < 0 || HD < 0) return DATTN_ERR_INVALID_ARGUMENT;
  if (dtype != DATTN_F32 && dtype != DATTN_F16 && dtype != DATTN_BF16) return DATTN_ERR_UNSUPPORTED;
  if (n_rel == 0 || HD == 0) return DATTN_OK;
  if (!E || !Wq || !Wk || !qr || !kr) return DATTN_ERR_INVALID_ARGUMENT;
  if (ld_e < hidden || ld_w < hidden || ld_out < HD) return DATTN_ERR_INVALID_ARGUMENT;
  if (hidden == 0 || hidden % 16) return DATTN_ERR_UNSUPPORTED;
  const int es = esize_of(dtype);
  if (!aligned16(E) || !aligned16(Wq) || !aligned16(Wk)) return DATTN_ERR_UNSUPPORTED;
  if ((ld_e * es) % 16 || (ld_w * es) % 16) return DATTN_ERR_UNSUPPORTED;
  // outputs and biases are accessed one element at a time
  const auto elem_ok = [es](const void* ptr) {
    return ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) % (uintptr_t)es) == 0;
  };
  if (!elem_ok(qr) || !elem_ok(kr) || !elem_ok(bq) || !elem_ok(bk)) return DATTN_ERR_UNSUPPORTED;
  return dattn::launch_rel_proj(E, ld_e, Wq, Wk, ld_w, bq, bk, qr, kr, ld_out, n_rel, hidden, HD,
                                dtype, stream);
}

const char* dattn_strerror(int status) {
  switch (status) {
    case DATTN_OK: return "ok";
    case DATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case DATTN_ERR_HIP: return "HIP launch failure";
    case DATTN_ERR_SCRATCH_TOO_SMALL:
      return "the problem needs more workspace than the allocation-free entry point's fixed "
             "device array holds (DATTN_NOALLOC_SCRATCH_BYTES); use dattn_bwd_varlen with a workspace";
    default: return "unknown status";
  }
}

}  // extern "C"
