/*
 * dattn.h - C ABI of libdattn.so, the disentangled-attention forward for
 * AMD Instinct MI355X (gfx950), with the steps around it: the relative-row
 * table, the per-head relative projections, and padded <-> packed rows.
 *
 * The operation is the exact, bidirectional DeBERTa-v2/v3 attention that
 * DisentangledFlash describes (README "Status": C2P/P2C disentangled
 * attention, FP16/BF16/strict FP32, head dims 32/64/128, factorised 2-D
 * padding masks, lengths up to 8192, packed cu_seqlens inference;
 * kernels-community discussion #31 "Motivation": same operation as the
 * reference encoder, no approximation, never materialising [B, H, L, L]).
 * For one sequence and one head, with positions i (query) and j (key):
 *
 *   S_ij = scale * ( q_i . k_j
 *                    + [flags & DATTN_C2P] q_i . kr[T(i - j)]
 *                    + [flags & DATTN_P2C] k_j . qr[T(j - i)] )
 *   O_i  = sum_j softmax_j(S_ij over valid keys) v_j
 *
 * T is the relative-row table written by rel_bucket(). The pages do not
 * print these formulas; they are the DeBERTa-v2/v3 definitions the README's
 * "Attribution" section refers to.
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers, owned by the caller. The
 *     library allocates nothing, keeps no state between calls and is
 *     re-entrant; calls on different streams may run concurrently.
 *   - Every call is asynchronous on `stream` (0 = the null stream) and never
 *     synchronises with the host. A DATTN_OK return means the work was
 *     enqueued.
 *   - Element types (dtype): DATTN_F32, DATTN_F16, DATTN_BF16. q, k, v, qr,
 *     kr and out all use the same type. Accumulation is in fp32. For the
 *     16-bit types the softmax weights are rounded to the element type
 *     before the P.V product, and on key tiles beyond the table's two
 *     saturation distances the forward forms the operand
 *     (q_i + qr[edge row]) * scale * log2(e) in fp32 and rounds it once to
 *     the element type (q_i * scale * log2(e) without P2C). With fp16 and a
 *     caller scale above ~0.69 that product can leave fp16's range where
 *     q_i + qr[row] alone would not; the default scales shrink it.
 *   - Head h of a token row occupies columns h*d .. h*d+d-1.
 *   - Row strides (ld_*) are in elements, must be >= H*d and a multiple of
 *     16 bytes; every array pointer must be 16-byte aligned. A fused QKV
 *     buffer [tokens, 3*H*d] is passed as three pointers with ld = 3*H*d.
 *     The row-copy entries (dattn_pack_rows, dattn_unpack_rows) are the
 *     exception: they move rows as bytes and take byte strides.
 *   - int32 arrays (tables, cu_seqlens, packing metadata) must be 4-byte
 *     aligned (UNSUPPORTED otherwise).
 *   - No hidden fallback: an unsupported case returns DATTN_ERR_UNSUPPORTED
 *     and the caller decides what to do.
 */
#ifndef DATTN_H
#define DATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DATTN_OK                    0
#define DATTN_ERR_INVALID_ARGUMENT  1  /* null pointer, bad size, inconsistent lengths */
#define DATTN_ERR_UNSUPPORTED       2  /* d, dtype, length > 8192, alignment or stride */
#define DATTN_ERR_HIP               3  /* a HIP launch failed */
#define DATTN_ERR_SCRATCH_TOO_SMALL 4  /* dattn_bwd_varlen_noalloc: problem exceeds its fixed array */

/* element types */
#define DATTN_F32   0
#define DATTN_F16   1
#define DATTN_BF16  2

/* position terms (flags bitfield) */
#define DATTN_C2P   1u   /* content-to-position: q_i . kr[T(i - j)] */
#define DATTN_P2C   2u   /* position-to-content: k_j . qr[T(j - i)] */

/* longest sequence (the README's bounded kernel families stop at 8192) */
#define DATTN_MAX_SEQLEN 8192

/*
 * rel_bucket - write the relative-row table T.
 *
 * rel_idx[r + max_len - 1] = clamp(b(r) + s, 0, 2s - 1) for every signed
 * distance r in [-(max_len-1), max_len-1], i.e. 2*max_len - 1 int32 entries.
 *   position_buckets > 0 : DeBERTa-v2 log buckets, mid = position_buckets/2,
 *       b(r) = r for |r| <= mid, else
 *       sign(r) * (mid + ceil((mid-1) ln(|r|/mid) / ln((M-1)/mid)))
 *       with M = max_relative_positions; s = position_buckets.
 *   position_buckets <= 0: no bucketing, b(r) = r, s = max_relative_positions.
 * The forward then reads 2s rows of qr and kr (n_rel = 2s).
 * The ceiling is of the real number, decided exactly: the kernel's float64
 * evaluation is used where it lies more than 1e-9 from an integer (its
 * error is below 1e-10 in the supported domain); the few distances closer
 * than that are decided on the host, before the launch, by an exact
 * comparison of integer powers, and passed to the kernel.
 *
 * rel_idx : device int32[2*max_len - 1], written.
 * Errors  : INVALID_ARGUMENT for rel_idx == NULL, max_len < 1, or bucket
 *           parameters where the formula is undefined (position_buckets == 1,
 *           or max_relative_positions - 1 <= position_buckets/2 when
 *           bucketing, or max_relative_positions < 1 without);
 *           UNSUPPORTED for max_len > 65536, position_buckets > 4096, or
 *           more than 32 near-integer distances (none is known to occur);
 *           HIP_ERROR if the launch fails.
 */
int rel_bucket(int32_t* rel_idx, int32_t max_len, int32_t position_buckets,
               int32_t max_relative_positions, hipStream_t stream);

/*
 * dattn_fwd_padded - forward over a right- or arbitrarily-padded batch.
 *
 * q, k, v : [B, L, >=H*d] token rows with stride ld_q / ld_k / ld_v elements;
 *           batch b starts at element b*L*ld.
 * qr, kr  : [n_rel, >=H*d] projected relative tables, row stride ld_rel,
 *           shared by the whole batch. May be NULL when flags == 0.
 * rel_idx : int32[2*rel_max_len - 1], the table from rel_bucket() for
 *           max_len = rel_max_len; needs rel_max_len >= L. The entries
 *           must be non-decreasing in the distance, as rel_bucket writes
 *           them (the kernels find the table's two saturation distances by
 *           search; other tables give undefined results). An entry outside
 *           [0, n_rel) reads the nearest edge row: below 0 row 0, at or
 *           above n_rel row n_rel - 1. May be NULL when flags == 0.
 * mask    : [B, L] bytes, nonzero = valid token, or NULL (all valid). It is
 *           the factorised 2-D mask m_i * m_j: a valid query attends to the
 *           valid keys only; positions are padded-row indices.
 * out     : [B, L, H*d], contiguous, written completely: rows of padded
 *           queries (m_i = 0) are zero.
 * flags   : DATTN_C2P | DATTN_P2C (0 gives plain softmax attention).
 * scale   : > 0 overrides the default 1/sqrt(d * (1 + #terms enabled)).
 *
 * Errors: INVALID_ARGUMENT (null pointer, B < 0, L < 0, H < 1, ld < H*d,
 * rel_max_len < L or n_rel < 1 when flags != 0, unknown flag bits, NaN
 * scale); UNSUPPORTED (d not 32/64/128, unknown dtype, L > 8192,
 * misaligned pointer or stride, relative tables of n_rel * ld_rel elements
 * spanning more than 2^31 - 1 bytes); HIP_ERROR. B*L == 0 is a no-op.
 */
int dattn_fwd_padded(const void* q, const void* k, const void* v,
                     int64_t ld_q, int64_t ld_k, int64_t ld_v,
                     const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                     const int32_t* rel_idx, int32_t rel_max_len,
                     const uint8_t* mask, void* out,
                     int32_t B, int32_t L, int32_t H, int32_t d, int32_t dtype,
                     uint32_t flags, float scale, hipStream_t stream);

/*
 * dattn_fwd_varlen - forward over packed sequences (FlashAttention-style
 * layout: README "Packed unpadded inference"; int32 cumulative lengths as
 * in the fold-attention README's packed self-attention).
 *
 * q, k, v    : [total_tokens, >=H*d] rows with strides ld_q / ld_k / ld_v.
 * cu_seqlens : device int32[nseq + 1], non-decreasing, cu[0] = 0,
 *              cu[nseq] = total_tokens. Sequence b is rows cu[b] ..
 *              cu[b+1]-1; its positions restart at 0. Zero-length
 *              sequences are allowed. Inconsistent values are undefined
 *              behaviour, but device reads stay clamped to total_tokens.
 * max_seqlen : host-side bound on every length (<= 8192, <= rel_max_len
 *              when flags != 0). nseq, max_seqlen and total_tokens are host
 *              values, so the call needs no device-to-host read. It also
 *              picks the tile height: 64 queries per workgroup for 16-bit
 *              types at d <= 64 when max_seqlen <= 128, else 128.
 * out        : [total_tokens, H*d], contiguous; every row is written.
 * Other arguments as for dattn_fwd_padded.
 *
 * Errors: as dattn_fwd_padded, with max_seqlen in place of L; nseq < 0 or
 * total_tokens < 0 is INVALID_ARGUMENT; nseq == 0 or total_tokens == 0 is
 * a no-op.
 */
int dattn_fwd_varlen(const void* q, const void* k, const void* v,
                     int64_t ld_q, int64_t ld_k, int64_t ld_v,
                     const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                     const int32_t* rel_idx, int32_t rel_max_len,
                     const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                     int64_t total_tokens, void* out,
                     int32_t H, int32_t d, int32_t dtype,
                     uint32_t flags, float scale, hipStream_t stream);

/*
 * dattn_fwd_padded_lse, dattn_fwd_varlen_lse - the same forwards, also
 * writing each row's log-sum-exp, the statistic a backward pass or a merge
 * of partial attentions reads:
 *
 *   lse[t * H + h] = ln sum_j exp(S_tj)   over the valid keys j of row t,
 *
 * with S the scaled scores above; -inf for rows with no valid key (padded
 * queries, empty sequences). lse is a device float32 array of [B*L, H]
 * (padded) or [total_tokens, H] (packed) entries, 4-byte aligned, written
 * for every row the output covers. Other arguments, outputs and errors are
 * those of dattn_fwd_padded / dattn_fwd_varlen; a NULL lse is
 * INVALID_ARGUMENT.
 */
int dattn_fwd_padded_lse(const void* q, const void* k, const void* v,
                         int64_t ld_q, int64_t ld_k, int64_t ld_v,
                         const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                         const int32_t* rel_idx, int32_t rel_max_len,
                         const uint8_t* mask, void* out, float* lse,
                         int32_t B, int32_t L, int32_t H, int32_t d, int32_t dtype,
                         uint32_t flags, float scale, hipStream_t stream);

int dattn_fwd_varlen_lse(const void* q, const void* k, const void* v,
                         int64_t ld_q, int64_t ld_k, int64_t ld_v,
                         const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                         const int32_t* rel_idx, int32_t rel_max_len,
                         const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                         int64_t total_tokens, void* out, float* lse,
                         int32_t H, int32_t d, int32_t dtype,
                         uint32_t flags, float scale, hipStream_t stream);

/*
 * dattn_fwd_padded_f32fast, dattn_fwd_varlen_f32fast - the forward on fp32
 * operands in the fast fp32 mode the DisentangledFlash README ("Status")
 * lists beside strict fp32. CDNA4 has no TF32 matrix instruction; the fp16
 * MFMA takes operands with TF32's 10-bit mantissa and accumulates in fp32.
 * So q, k, v (and qr, kr with position terms) are rounded once to fp16
 * (nearest even) into the workspace, the fp16 forward runs on them, and its
 * output (rounded to fp16 like any fp16 output) is widened into the fp32
 * out. Accuracy is that of the fp16 forward; the exponent range is fp16's
 * (magnitudes above 65504 overflow, below 2^-24 flush to zero).
 *
 * Arguments as for dattn_fwd_padded / dattn_fwd_varlen with dtype fixed
 * to fp32 (q, k, v, qr, kr, out are float), plus:
 * workspace : device memory of at least dattn_fwd_f32fast_workspace_size()
 *             bytes for `rows` = B*L (padded) or total_tokens (packed) and
 *             n_rel (0 when flags == 0); 16-byte aligned, owned by the
 *             caller, overwritten; calls that share a workspace must not
 *             overlap.
 * Errors: those of the fp32 forward, plus INVALID_ARGUMENT for a NULL or
 * too small workspace, UNSUPPORTED for a misaligned one.
 */
int64_t dattn_fwd_f32fast_workspace_size(int64_t rows, int32_t n_rel, int32_t H, int32_t d);

int dattn_fwd_padded_f32fast(const void* q, const void* k, const void* v,
                             int64_t ld_q, int64_t ld_k, int64_t ld_v,
                             const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                             const int32_t* rel_idx, int32_t rel_max_len,
                             const uint8_t* mask, void* out,
                             int32_t B, int32_t L, int32_t H, int32_t d,
                             uint32_t flags, float scale,
                             void* workspace, int64_t workspace_bytes, hipStream_t stream);

int dattn_fwd_varlen_f32fast(const void* q, const void* k, const void* v,
                             int64_t ld_q, int64_t ld_k, int64_t ld_v,
                             const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                             const int32_t* rel_idx, int32_t rel_max_len,
                             const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                             int64_t total_tokens, void* out, int32_t H, int32_t d,
                             uint32_t flags, float scale,
                             void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * Backward of the forward above: the gradients of a scalar loss with respect
 * to q, k, v and the relative tables qr, kr, given dout = dLoss/dout. The
 * pages' forward is inference-only (DisentangledFlash README "Status"); the
 * kernels-community discussion #31 ("Packaging and validation") names the
 * backward as the next step. With P the softmax weights (recomputed from the
 * forward's log-sum-exp), D_i = dout_i . out_i and S the scaled scores:
 *
 *   dv_j   = sum_i P_ij dout_i
 *   dS_ij  = P_ij (dout_i . v_j - D_i)            (0 for masked pairs)
 *   dq_i   = scale sum_j dS_ij (k_j + [C2P] kr[T(i - j)])
 *   dk_j   = scale sum_i dS_ij (q_i + [P2C] qr[T(j - i)])
 *   dkr[r] = scale sum over pairs with T(i - j) = r of dS_ij q_i   [C2P]
 *   dqr[r] = scale sum over pairs with T(j - i) = r of dS_ij k_j   [P2C]
 *
 * dkr and dqr collect every sequence of the batch (the tables are shared).
 * The result is deterministic: every output element is produced by one
 * thread from a reduction in a fixed order (no atomics), so repeated calls
 * give identical bits.
 *
 * rel_bucket_band - the band of rel_bucket's table: the least W >= 1 such
 * that every entry at a distance >= W equals the table's last entry and every
 * entry at a distance <= -W its first (host computation, no device work);
 * -1 for parameters rel_bucket rejects. For DeBERTa's 256/512 buckets it is
 * 512 once max_len exceeds 512 (the last row is reached from distance 506
 * on, the first only from -512 on).
 */
int32_t rel_bucket_band(int32_t max_len, int32_t position_buckets, int32_t max_relative_positions);

/*
 * dattn_bwd_workspace_size - bytes of device workspace the backward needs
 * for total_tokens rows (B*L for the padded layout), nseq sequences (B for
 * the padded layout), H heads of d, the element type and the band; -1 for
 * invalid arguments. The workspace holds per-row statistics, fp32 partial
 * dq/dk, and the dS of the pairs closer than `band` stored by distance
 * (H * (2*band - 1) * total_tokens elements); with flags == 0 use band = 1.
 */
int64_t dattn_bwd_workspace_size(int64_t total_tokens, int32_t nseq, int32_t H, int32_t d,
                                 int32_t dtype, int32_t band);

/*
 * dattn_bwd_padded, dattn_bwd_varlen - the backward.
 *
 * q, k, v, qr, kr, rel_idx, rel_max_len, mask / cu_seqlens, nseq,
 *   max_seqlen, total_tokens, H, d, dtype, flags, scale: exactly as given to
 *   the forward (dattn_fwd_padded_lse / dattn_fwd_varlen_lse).
 * out, lse   : the forward's output and log-sum-exp of the same call;
 *              out rows at stride ld_o.
 * dout       : [rows, >=H*d] gradient of the output, stride ld_do.
 * band       : W >= 1 such that rel_idx is constant beyond +-W (entries at
 *              distances >= W equal its last entry, at <= -W its first), at
 *              most rel_max_len; rel_bucket_band() gives it for rel_bucket's
 *              tables, rel_max_len is always valid. Ignored when flags == 0.
 * dq, dk, dv : [rows, H*d] contiguous, written completely (zero rows for
 *              padded positions).
 * dqr, dkr   : [n_rel, H*d] contiguous, written completely (rows no pair
 *              reads are zero; a disabled term's table gradient is zero).
 *              May be NULL when flags == 0.
 * workspace  : device memory of at least dattn_bwd_workspace_size() bytes,
 *              16-byte aligned, owned by the caller, overwritten; calls
 *              that share a workspace must not overlap.
 *
 * Errors: those of the forward, plus INVALID_ARGUMENT for a NULL out, dout,
 * lse, dk, dv, workspace (or dqr/dkr with flags != 0), ld_o / ld_do < H*d,
 * band outside [1, rel_max_len] with flags != 0, or a workspace smaller
 * than required; UNSUPPORTED for misaligned pointers or strides.
 */
int dattn_bwd_padded(const void* q, const void* k, const void* v,
                     int64_t ld_q, int64_t ld_k, int64_t ld_v,
                     const void* out, const void* dout, int64_t ld_o, int64_t ld_do,
                     const float* lse,
                     const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                     const int32_t* rel_idx, int32_t rel_max_len, int32_t band,
                     const uint8_t* mask, void* dq, void* dk, void* dv, void* dqr, void* dkr,
                     void* workspace, int64_t workspace_bytes,
                     int32_t B, int32_t L, int32_t H, int32_t d, int32_t dtype,
                     uint32_t flags, float scale, hipStream_t stream);

int dattn_bwd_varlen(const void* q, const void* k, const void* v,
                     int64_t ld_q, int64_t ld_k, int64_t ld_v,
                     const void* out, const void* dout, int64_t ld_o, int64_t ld_do,
                     const float* lse,
                     const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                     const int32_t* rel_idx, int32_t rel_max_len, int32_t band,
                     const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                     int64_t total_tokens, void* dq, void* dk, void* dv, void* dqr, void* dkr,
                     void* workspace, int64_t workspace_bytes,
                     int32_t H, int32_t d, int32_t dtype,
                     uint32_t flags, float scale, hipStream_t stream);

/*
 * dattn_bwd_varlen_noalloc - dattn_bwd_varlen without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The workspace is a fixed device array of DATTN_NOALLOC_SCRATCH_BYTES
 * inside the library: one copy per GPU, held from the library's load until
 * the process ends. The call allocates nothing (no hipMalloc, no allocating
 * library routine); it uses the array of the current device, so the stream
 * must belong to the current device. Every argument has the meaning it has
 * in dattn_bwd_varlen, and the outputs are identical to its outputs.
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (no call reads a cell it has not written first): two calls that
 * overlap on one GPU, on different streams or host threads, race and give
 * wrong results. Serialise them.
 *
 * Errors: those of dattn_bwd_varlen, plus DATTN_ERR_SCRATCH_TOO_SMALL when
 * dattn_bwd_workspace_size() of the problem exceeds
 * DATTN_NOALLOC_SCRATCH_BYTES (checked before any HIP call), and
 * DATTN_ERR_HIP if the array's device address cannot be looked up.
 */
#define DATTN_NOALLOC_SCRATCH_BYTES (128ll << 20)

int dattn_bwd_varlen_noalloc(const void* q, const void* k, const void* v,
                             int64_t ld_q, int64_t ld_k, int64_t ld_v,
                             const void* out, const void* dout, int64_t ld_o, int64_t ld_do,
                             const float* lse,
                             const void* qr, const void* kr, int64_t ld_rel, int32_t n_rel,
                             const int32_t* rel_idx, int32_t rel_max_len, int32_t band,
                             const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                             int64_t total_tokens, void* dq, void* dk, void* dv, void* dqr,
                             void* dkr, int32_t H, int32_t d, int32_t dtype,
                             uint32_t flags, float scale, hipStream_t stream);

/*
 * dattn_rel_proj - the per-head relative tables from the relative embeddings:
 *
 *   qr = E Wq^T + bq,   kr = E Wk^T + bk
 *
 * In DeBERTa-v2/v3 (the models the DisentangledFlash README's "Attribution"
 * section names) qr and kr are the attention layer's query and key linear
 * maps applied to the relative-embedding table that the whole batch
 * shares; the forward then reads their rows through rel_idx.
 *
 * E       : [n_rel, hidden] relative embeddings, row stride ld_e.
 * Wq, Wk  : [HD, hidden] weights in nn.Linear layout (one output feature per
 *           row), row stride ld_w; HD = H*d.
 * bq, bk  : [HD] biases, or NULL (zero).
 * qr, kr  : [n_rel, HD] outputs, row stride ld_out; exactly the arrays
 *           dattn_fwd_padded / dattn_fwd_varlen take (n_rel rows).
 * All arrays have element type dtype; products accumulate in fp32 and each
 * output is rounded once. One launch on `stream` writes both tables.
 *
 * Errors: INVALID_ARGUMENT (negative size, NULL array when n_rel*HD > 0,
 * ld_e or ld_w < hidden, ld_out < HD); UNSUPPORTED (dtype, hidden not a
 * positive multiple of 16, E/Wq/Wk not 16-byte aligned or their strides not
 * multiples of 16 bytes, qr/kr/bq/bk not aligned to the element size);
 * HIP_ERROR. n_rel == 0 or HD == 0 is a no-op.
 */
int dattn_rel_proj(const void* E, int64_t ld_e, const void* Wq, const void* Wk, int64_t ld_w,
                   const void* bq, const void* bk, void* qr, void* kr, int64_t ld_out,
                   int32_t n_rel, int32_t hidden, int32_t HD, int32_t dtype, hipStream_t stream);

/*
 * Packing a padded batch for dattn_fwd_varlen and back (DisentangledFlash
 * README, "Packed unpadded inference": right-padded hidden states and their
 * attention mask become FlashAttention-style [total_tokens, width] rows with
 * int32 cu_seqlens; the metadata is reused by every encoder layer, and the
 * packed outputs are returned to the padded layout). The README's benchmark
 * notes that packing has a fixed cost, so it pays once padding is heavy.
 *
 * dattn_pack_index - build the packing metadata of a [B, L] mask.
 *
 * mask          : [B, L] bytes, nonzero = valid token, or NULL (all valid).
 *                 Any pattern is accepted; valid tokens keep their order.
 * cu_seqlens    : device int32[B + 1], written: cu[0] = 0 and cu[b+1] - cu[b]
 *                 = valid tokens of row b. For a right-padded mask this is
 *                 exactly the cu_seqlens dattn_fwd_varlen takes.
 * token_rows    : device int32[B * L], written: entry r < cu[B] is the padded
 *                 row b*L + l of the r-th valid token (row-major order);
 *                 entries from cu[B] on are -1.
 * row_to_packed : device int32[B * L], written: the packed index of padded
 *                 row i, or -1 where the mask is zero.
 * max_seqlen    : device int32[1] written with the longest row, or NULL.
 * Work is one launch on `stream` for B <= 4096 rows and B*L <= 2^18
 * tokens (one workgroup builds the whole index), three launches above
 * that (per-row ranks, a scan, the placement); nothing is read back to the
 * host, so
 * a caller that needs cu[B] (to size the packed buffers) or max_seqlen on
 * the host copies them itself. L is always a valid max_seqlen bound.
 *
 * Errors: INVALID_ARGUMENT (B < 0, L < 0, cu_seqlens NULL, or token_rows /
 * row_to_packed NULL with B*L > 0); UNSUPPORTED (B*L > 2^31 - 1 or
 * B = 2^31 - 1); HIP_ERROR. B == 0 writes cu[0] = 0 only.
 */
int dattn_pack_index(const uint8_t* mask, int32_t B, int32_t L, int32_t* cu_seqlens,
                     int32_t* token_rows, int32_t* row_to_packed, int32_t* max_seqlen,
                     hipStream_t stream);

/*
 * dattn_pack_rows - dst[r] = src[token_rows[r]] for r < n_rows.
 *
 * Rows are opaque bytes (any element type; a fused QKV row packs in one
 * call). src has n_src rows of row_bytes bytes at stride ld_src_bytes; dst
 * rows are at stride ld_dst_bytes. An index outside [0, n_src) (the -1
 * tail of token_rows) leaves dst row r untouched, so with n_rows = B*L only
 * the first cu[B] rows of dst are written and dst needs only that many.
 *
 * dattn_unpack_rows - dst[i] = src[row_to_packed[i]], or a zero row where
 * the index is outside [0, n_src), for i < n_rows: every row of dst is
 * written, padding rows with zeros.
 *
 * Both: pointers 16-byte aligned; row_bytes and both strides multiples of
 * 16 bytes, strides >= row_bytes; src and dst must not overlap. Errors:
 * INVALID_ARGUMENT (negative size or count, NULL pointer with n_rows > 0
 * and row_bytes > 0, stride < row_bytes); UNSUPPORTED (alignment, a size
 * not a multiple of 16 bytes); HIP_ERROR. n_rows == 0 or row_bytes == 0 is
 * a no-op.
 */
int dattn_pack_rows(const void* src, int64_t ld_src_bytes, int64_t n_src,
                    const int32_t* token_rows, int64_t n_rows, int64_t row_bytes, void* dst,
                    int64_t ld_dst_bytes, hipStream_t stream);

int dattn_unpack_rows(const void* src, int64_t ld_src_bytes, int64_t n_src,
                      const int32_t* row_to_packed, int64_t n_rows, int64_t row_bytes, void* dst,
                      int64_t ld_dst_bytes, hipStream_t stream);

/* Static, human-readable text for a status code. */
const char* dattn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* DATTN_H */
