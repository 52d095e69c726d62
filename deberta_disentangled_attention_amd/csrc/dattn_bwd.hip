// Backward of the disentangled-attention forward for gfx950 (MI355X).
//
// The forward (DisentangledFlash README "Status": inference only; the
// kernels-community discussion #31 "Packaging and validation" announces a
// backward) computes, for one sequence and head,
//   S_ij = tau (q_i.k_j + [C2P] q_i.kr[T(i-j)] + [P2C] k_j.qr[T(j-i)]),
//   P = softmax over the valid keys of each row, O = P V.
// Its gradients, with D_i = dO_i . O_i and P recomputed from the forward's
// row log-sum-exp:
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dQ_i  = tau sum_j dS_ij (k_j + [C2P] kr[T(i-j)])
//   dK_j  = tau sum_i dS_ij (q_i + [P2C] qr[T(j-i)])
//   dkr_r = tau sum of dS_ij q_i over the pairs with T(i-j) = r      [C2P]
//   dqr_r = tau sum of dS_ij k_j over the pairs with T(j-i) = r      [P2C]
// dkr and dqr collect every sequence of the batch.
//
// Decomposition (deterministic: every output element is written by one
// thread after a reduction in a fixed order; no atomics):
//  1. dsum: D_i per row and head.
//  2. main<Q side>: a workgroup owns 128 queries of one (sequence, head) and
//     walks the keys in blocks of 32. It recomputes S (with the position
//     terms: beyond the band from the table's saturated rows, inside it as
//     the forward's band path, per wave E = kr-row x q and F = k x qr-row
//     products gathered along the diagonal through LDS), P and dS,
//     accumulates the content part of dQ (dS K) and, per query, the sums of
//     dS over the pairs whose distance u = i - j lies beyond the band
//     (|u| >= band, where the table is constant); the dS of pairs inside
//     the band go to a store indexed by (distance, query token), Dq.
//  3. main<K side>: a workgroup owns 128 keys and walks the queries. The
//     score is symmetric under exchanging (q, kr) with (k, qr) and i with j,
//     so the same tile routine with those operands exchanged yields S in
//     the key-major layout; it accumulates dV, the content part of dK, the
//     per-key sums beyond the band and the store indexed by (distance, key
//     token), Dk.
//  4. pos_grad: the position parts of dQ (Dq with kr rows) and dK (Dk with
//     qr rows) as MFMA products, plus the beyond-band sums times the
//     table's end rows; each output row is rounded once.
//  5. pos_w: per (sequence, head) and distance, W_u = sum_i Dq[u][i] q_i and
//     sum_j Dk[u][j] k_j (MFMA), and (pos_farw) the beyond-band sums times
//     q or k.
//  6. pos_rel: dkr / dqr rows, summing W over the sequences in order and
//     over the distances that map to each row.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dattn_device.h"
#include "dattn_internal.h"

namespace dattn {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kBwdMaxSeqLen = 8192;

template <class T, int D>
struct BCfg {
  static constexpr int ES = Ty<T>::ESIZE;
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BX = 32 * NW;                 // lane-side positions per workgroup
  static constexpr int BY = 32;                      // other-side positions per block
  static constexpr int HALF = D / 2;
  static constexpr int NU = HALF * ES / 16;          // 16-byte units per lane half-row
  static constexpr int NC = HALF / Ty<T>::LANE_K;    // MFMAs per d-long product
  static constexpr int NDB = D / 32;
  static constexpr int UPR = D * ES / 16;            // 16-byte units per row
  static constexpr int EPU = 16 / ES;
  static constexpr int RPITCH = D + EPU;             // staged row pitch (elements)
  static constexpr int ROWS_BYTES = BY * RPITCH * ES;
  static constexpr int NPF = (BY * UPR + NT - 1) / NT;   // 16-byte units per thread per staged block
  // rows of the next block are loaded while the current one is computed,
  // except where their registers do not fit (fp32, d = 128)
  static constexpr bool PREFETCH = !(ES == 4 && D == 128);
  static constexpr int SCR_BYTES = 64 * 32 * 4;      // per wave: 64 distances x 32 positions
  // LDS: two row blocks, per-wave scratch, per-y stats
  static constexpr int OFF_R1 = 0;
  static constexpr int OFF_R2 = OFF_R1 + ROWS_BYTES;
  static constexpr int OFF_SCR = OFF_R2 + ROWS_BYTES;
  static constexpr int CARRY_BYTES = 31 * 32 * 4;    // per wave: distance-store rows awaiting the next block
  static constexpr int OFF_CARRY = OFF_SCR + NW * SCR_BYTES;
  static constexpr int OFF_XF = OFF_CARRY + NW * CARRY_BYTES;   // per lane: the far-block operand
  static constexpr int OFF_STAT = OFF_XF + NT * NU * 16;
  static constexpr int OFF_MISC = OFF_STAT + 2 * BY * 4;
  static constexpr int LDS_BYTES = OFF_MISC + 64;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert((ROWS_BYTES % 16) == 0, "alignment");
};

__device__ __forceinline__ int64_t unit_base(const BwdParams& p, int b) {
  return p.cu_seqlens ? (int64_t)p.cu_seqlens[b] : (int64_t)b * p.L;
}
__device__ __forceinline__ int unit_len(const BwdParams& p, int b) {
  if (p.cu_seqlens) {
    const int64_t c0 = min((int64_t)p.cu_seqlens[b], p.tokens);
    const int64_t c1 = min(max((int64_t)p.cu_seqlens[b + 1], c0), p.tokens);
    return (int)min(c1 - c0, (int64_t)kBwdMaxSeqLen);
  }
  return p.L;
}

template <class T>
__device__ __forceinline__ float to_f(const void* base, int64_t idx) {
  if constexpr (std::is_same<T, TF32>::value) return reinterpret_cast<const float*>(base)[idx];
  else if constexpr (std::is_same<T, TF16>::value) return (float)reinterpret_cast<const _Float16*>(base)[idx];
  else return (float)reinterpret_cast<const __bf16*>(base)[idx];
}
template <class T>
__device__ __forceinline__ void from_f(void* base, int64_t idx, float x) {
  if constexpr (std::is_same<T, TF32>::value) reinterpret_cast<float*>(base)[idx] = x;
  else if constexpr (std::is_same<T, TF16>::value) reinterpret_cast<_Float16*>(base)[idx] = (_Float16)x;
  else reinterpret_cast<__bf16*>(base)[idx] = (__bf16)x;
}

// table row of a signed distance, clamped into [0, n_rel)
__device__ __forceinline__ int rel_row(const BwdParams& p, int dist) {
  const int R = p.rel_max_len;
  int x = dist + R - 1;
  x = x < 0 ? 0 : (x > 2 * R - 2 ? 2 * R - 2 : x);
  const int r = p.rel_idx[x];
  return r < 0 ? 0 : (r >= p.n_rel ? p.n_rel - 1 : r);
}

// ---------------------------------------------------------------------------
// 1. D_i = dO_i . O_i
// ---------------------------------------------------------------------------

template <class T>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(BwdParams p, int d) {
  constexpr int EPU = 16 / Ty<T>::ESIZE;   // elements per 16-byte unit
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t rows = p.tokens * p.H;
  const unsigned char* dob = reinterpret_cast<const unsigned char*>(p.dout);
  const unsigned char* ob = reinterpret_cast<const unsigned char*>(p.o);
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < rows; idx += stride) {
    const int64_t t = idx / p.H;
    const int h = (int)(idx - t * p.H);
    const unsigned char* a = dob + (t * p.ld_do + (int64_t)h * d) * Ty<T>::ESIZE;
    const unsigned char* b = ob + (t * p.ld_o + (int64_t)h * d) * Ty<T>::ESIZE;
    float acc = 0.f;
    for (int e = 0; e < d; e += EPU) acc += dot16<T>(ld16(a + e * Ty<T>::ESIZE), ld16(b + e * Ty<T>::ESIZE));
    p.dsum[idx] = acc;
  }
}

// ---------------------------------------------------------------------------
// 2./3. the tile loops
// ---------------------------------------------------------------------------

// A block of BY rows (positions y0 .. y0+BY-1 of the unit; rows of
// positions past the extent or masked are zero) as 16-byte units, NPF per
// thread: loaded into registers one block ahead, stored to LDS row-major
// (pitch RPITCH) when the block's turn comes.
template <class T, int D>
__device__ __forceinline__ void load_rows(uint4* r, const unsigned char* g, int64_t ld,
                                          int64_t tok0, int y0, int ext, const uint8_t* mrow, int64_t hoff,
                                          int tid) {
  typedef BCfg<T, D> C;
#pragma unroll
  for (int k = 0; k < C::NPF; ++k) {
    const int x = tid + k * C::NT;
    const int row = x / C::UPR, u = x - row * C::UPR;
    const int y = y0 + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (x < C::BY * C::UPR && y < ext && (!mrow || mrow[y])) v = ld16(g + ((tok0 + y) * ld + hoff) * C::ES + 16 * u);
    r[k] = v;
  }
}

template <class T, int D>
__device__ __forceinline__ void store_rows(const uint4* r, unsigned char* rows, int tid) {
  typedef BCfg<T, D> C;
#pragma unroll
  for (int k = 0; k < C::NPF; ++k) {
    const int x = tid + k * C::NT;
    const int row = x / C::UPR, u = x - row * C::UPR;
    if (x < C::BY * C::UPR) *reinterpret_cast<uint4*>(rows + row * C::RPITCH * C::ES + 16 * u) = r[k];
  }
}

// KSIDE = false: lanes own queries (x = i), the loop walks keys (y = j).
// KSIDE = true:  lanes own keys (x = j), the loop walks queries (y = i).
template <class T, int D, bool KSIDE, bool VARLEN>
// two workgroups per CU (two waves per SIMD) where the registers allow it
__global__ __launch_bounds__(256, (D <= 64 && Ty<T>::ESIZE == 2) ? 2 : 1) void bwd_main_kernel(BwdParams p) {
  typedef BCfg<T, D> C;
  constexpr int ES = C::ES;
  constexpr int NU = C::NU;
  constexpr int NC = C::NC;
  constexpr int NDB = C::NDB;
  constexpr int NT = C::NT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
  unsigned char* R1 = smem + C::OFF_R1;   // rows for S: keys (Q side) / queries (K side)
  unsigned char* R2 = smem + C::OFF_R2;   // rows for dP: V (Q side) / dO (K side)
  float* ystat = reinterpret_cast<float*>(smem + C::OFF_STAT);   // K side: lse, D of the block's queries
  int* misc = reinterpret_cast<int*>(smem + C::OFF_MISC);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  float* scr = reinterpret_cast<float*>(smem + C::OFF_SCR + wave * C::SCR_BYTES);

  // ---- item -> (unit, head, tile of 128 lane-side positions) ---------------
  int b, head, xt;
  const int item = blockIdx.x;
  if (!VARLEN) {
    const int per_b = p.H * p.n_qtiles;
    b = item / per_b;
    const int rest = item - b * per_b;
    head = rest / p.n_qtiles;
    xt = rest - head * p.n_qtiles;
  } else {
    head = item / p.n_qtiles;
    const int t = item - head * p.n_qtiles;
    const int64_t tot = p.tokens;
    const int32_t* cu = p.cu_seqlens;
    const int first_after = block_first_true<NT>(
        p.nseq, [&](int bb) { return min((int64_t)cu[bb], tot) / C::BX + bb > t; }, &misc[0], tid);
    b = max(first_after - 1, 0);
    xt = t - (int)(min((int64_t)cu[b], tot) / C::BX) - b;
  }
  const int len = unit_len(p, b);
  const int64_t tok0 = unit_base(p, b);
  // padded layout: positions past the last valid one are never visited
  int ext = len;
  const uint8_t* mrow = (!VARLEN && p.mask) ? p.mask + (int64_t)b * p.L : nullptr;
  if (mrow) {
    if (tid == 0) misc[1] = 0;
    __syncthreads();
    int last = 0;
    for (int j = tid; j < p.L; j += NT)
      if (mrow[j]) last = j + 1;
    if (last) atomicMax(&misc[1], last);
    __syncthreads();
    ext = misc[1];
    __syncthreads();
  }
  const int x0 = xt * C::BX;
  const int x0w = x0 + 32 * wave;
  const int x = x0w + li;
  const bool x_in = xt >= 0 && x < ext;
  const bool x_valid = x_in && (!mrow || mrow[x] != 0);
  const int64_t hoff = (int64_t)head * D;
  const float tau = p.tau;
  const bool c2p = (p.flags & 1u) != 0, p2c = (p.flags & 2u) != 0;
  // the "E" term reads the lane-side vector with table rows at T(x - y), the
  // "F" term the y-side rows with table rows at T(y - x)
  const bool e_on = KSIDE ? p2c : c2p;
  const bool f_on = KSIDE ? c2p : p2c;

  const unsigned char* Qg = reinterpret_cast<const unsigned char*>(p.q);
  const unsigned char* Kg = reinterpret_cast<const unsigned char*>(p.k);
  const unsigned char* Vg = reinterpret_cast<const unsigned char*>(p.v);
  const unsigned char* DOg = reinterpret_cast<const unsigned char*>(p.dout);
  const unsigned char* ERg = reinterpret_cast<const unsigned char*>(KSIDE ? p.qr : p.kr) + (hoff + lh * C::HALF) * ES;
  const unsigned char* FRg = reinterpret_cast<const unsigned char*>(KSIDE ? p.kr : p.qr) + (hoff + lh * C::HALF) * ES;
  const int64_t ld_rel_b = p.ld_rel * ES;

  if (xt < 0) return;   // packed: a slot before the sequence's first tile
  // positions x of the unit that take no part (past the extent, masked)
  // still get their rows written: zero gradients, zero sums beyond the band
  auto write_zero_row = [&]() {
    if (x >= len) return;
    const int64_t t = tok0 + x;
    float* part = KSIDE ? p.dk_part : p.dq_part;
    for (int dd = lh; dd < D; dd += 2) {
      part[(t * p.H + head) * D + dd] = 0.f;
      if (KSIDE) from_f<T>(p.dv, t * ((int64_t)p.H * D) + hoff + dd, 0.f);
    }
    if (lh == 0) {
      float* fs = KSIDE ? p.bfar : p.afar;
      fs[(t * p.H + head) * 2 + 0] = 0.f;
      fs[(t * p.H + head) * 2 + 1] = 0.f;
    }
  };
  // The distance store has no global clear: every in-band row of every
  // token of the unit is written by the wave that owns the token, by the
  // band blocks (put_rows below) or here, with zeros for the distances
  // outside [ulo, uhi] (ulo > uhi: all of them), whose pairs do not exist.
  const bool dg_on = KSIDE ? (p.flags & 2u) != 0 : (p.flags & 1u) != 0;
  auto zero_rows = [&](int ulo, int uhi) {
    using ZE = typename std::conditional<Ty<T>::ESIZE == 2, uint2, f32x4_t>::type;
    const int64_t tw0 = tok0 + x0w;
    unsigned char* base = reinterpret_cast<unsigned char*>(KSIDE ? p.dgk : p.dgq) +
                          ((int64_t)head * p.dg_groups + (tw0 >> 5)) * p.dg_rows * 32 * Ty<T>::ESIZE;
    const int nrows = 2 * p.band - 1;
    for (int j = lane; j < nrows * 8; j += 64) {
      const int u = j / 8 - (p.band - 1), c = j & 7;   // (distance, 4-token unit)
      if (u >= ulo && u <= uhi) continue;
      const int xl = x0w + 4 * c;
      const int tl = (int)(tw0 & 31) + 4 * c;
      if (((tw0 & 3) == 0) && xl + 3 < len) {
        *reinterpret_cast<ZE*>(base + (((tl >> 5) * p.dg_rows + (u + p.dg_rb)) * 32 + (tl & 31)) * Ty<T>::ESIZE) = ZE{};
      } else {
        for (int e = 0; e < 4 && xl + e < len; ++e) {
          const int te = tl + e;
          unsigned char* q = base + (((te >> 5) * p.dg_rows + (u + p.dg_rb)) * 32 + (te & 31)) * Ty<T>::ESIZE;
          if constexpr (Ty<T>::ESIZE == 2) *reinterpret_cast<uint16_t*>(q) = 0;
          else *reinterpret_cast<float*>(q) = 0.f;
        }
      }
    }
  };
  if (x0 >= ext) {   // uniform: no position of this tile takes part
    write_zero_row();
    if (dg_on && x0w < len) zero_rows(1, 0);
    return;
  }

  // lane-side operands (B operands of the products): the position's vector
  // for S, and dO (Q side) or v (K side) for dP
  uint4 xs[NU], xp[NU];
  {
    const unsigned char* gs = KSIDE ? Kg : Qg;
    const int64_t lds = KSIDE ? p.ld_k : p.ld_q;
    const unsigned char* gp = KSIDE ? Vg : DOg;
    const int64_t ldp = KSIDE ? p.ld_v : p.ld_do;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      xs[u] = x_valid ? ld16(gs + ((tok0 + x) * lds + hoff + lh * C::HALF) * ES + 16 * u) : make_uint4(0, 0, 0, 0);
      xp[u] = x_valid ? ld16(gp + ((tok0 + x) * ldp + hoff + lh * C::HALF) * ES + 16 * u) : make_uint4(0, 0, 0, 0);
    }
  }
  // P = exp2(S c1 - lse2) with c1 = tau log2(e) and lse2 = lse log2(e);
  // lse2 = +inf for rows that take no part or have no valid key (P = 0)
  const float l2e = 1.4426950408889634f;
  const float c1 = p.tau * l2e;
  const float kPosInf = __builtin_huge_valf();
  float lse2_x = kPosInf, d_x = 0.f;   // Q side: this query's
  if (!KSIDE && x_valid) {
    const float l = p.lse[(tok0 + x) * p.H + head];
    lse2_x = l == kNegInf ? kPosInf : l * l2e;
    d_x = p.dsum[(tok0 + x) * p.H + head];
  }

  // Blocks whose pairs all lie beyond the band (x - y >= band: "gt", or
  // <= -band: "lt") read one table row per term: the E term is the lane
  // scalar xs . ER[row] and the F term joins the S product through the
  // operand xs + FR[row] (formed in fp32, rounded once to the element
  // type). gt blocks come first in the loop, lt blocks last, so one operand
  // set is live at a time.
  const bool terms = e_on || f_on;
  const int row_top = terms ? rel_row(p, p.rel_max_len - 1) : 0;
  const int row_bot = terms ? rel_row(p, -(p.rel_max_len - 1)) : 0;
  unsigned char* xf_lds = smem + C::OFF_XF + tid * NU * 16;   // this lane's far operand
  float e_far = 0.f;
  auto make_far = [&](bool lt) {
    const int erow = lt ? row_bot : row_top, frow = lt ? row_top : row_bot;
    if (f_on) {
      uint4 rf[NU];
      load_half_row<NU>(rf, FRg + (int64_t)frow * ld_rel_b);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if constexpr (ES == 2) {
          const auto a = __builtin_bit_cast(typename Ty<T>::frag, xs[u]);
          const auto b = __builtin_bit_cast(typename Ty<T>::frag, rf[u]);
          f32x8_t sum;
#pragma unroll
          for (int e = 0; e < 8; ++e) sum[e] = (float)a[e] + (float)b[e];
          *reinterpret_cast<uint4*>(xf_lds + 16 * u) = __builtin_bit_cast(uint4, Ty<T>::cvt8(sum));
        } else {
          const f32x4_t a = __builtin_bit_cast(f32x4_t, xs[u]), b = __builtin_bit_cast(f32x4_t, rf[u]);
          *reinterpret_cast<uint4*>(xf_lds + 16 * u) = __builtin_bit_cast(uint4, a + b);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) *reinterpret_cast<uint4*>(xf_lds + 16 * u) = xs[u];
    }
    float e = 0.f;
    if (e_on) {
      uint4 rf[NU];
      load_half_row<NU>(rf, ERg + (int64_t)erow * ld_rel_b);
#pragma unroll
      for (int u = 0; u < NU; ++u) e += dot16<T>(xs[u], rf[u]);
      e += __shfl_xor(e, 32);
    }
    e_far = e;
  };
  bool far_lt_ready = false;
  if (terms) make_far(false);

  f32x16_t acc1[NDB], acc2[NDB];   // Q side: dQ^T; K side: dV^T (acc1), dK^T (acc2)
#pragma unroll
  for (int db = 0; db < NDB; ++db) { acc1[db] = f32x16_t{}; acc2[db] = f32x16_t{}; }
  float far_gt = 0.f, far_lt = 0.f;   // sums of dS over pairs with u >= band / u <= -band
  const int band = p.band;

  // A operand of the gradient products: a staged block read transposed
  // (m = the d index, the lane's; reduction over the block's positions y in
  // the order the dS / P registers hold them: 16c + 4lh + {0-3, 8-11} for
  // 16-bit types, 8c + 4lh + 0..3 for fp32)
  auto top = [&](const unsigned char* rows) {
    return [=](int c, int db) {
      if constexpr (ES == 2) {
        const int g = lane >> 4, t = lane & 15;
        const unsigned char* a =
            rows + ((16 * c + 4 * (g >> 1) + (t >> 2)) * C::RPITCH + 32 * db + 16 * (g & 1) + 4 * (t & 3)) * 2;
        const uint2 lo = lds_tr16(a), hi = lds_tr16(a + 8 * C::RPITCH * 2);
        return __builtin_bit_cast(typename Ty<T>::frag, make_uint4(lo.x, lo.y, hi.x, hi.y));
      } else {
        const float* r = reinterpret_cast<const float*>(rows) + (8 * c + 4 * lh) * C::RPITCH + 32 * db + li;
        return f32x4_t{r[0], r[C::RPITCH], r[2 * C::RPITCH], r[3 * C::RPITCH]};
      }
    };
  };
  // acc[db] += (transposed block)^T-operand x frag
  auto grad_acc = [&](f32x16_t (&acc)[NDB], auto op, const f32x16_t& g) {
    if constexpr (ES == 2) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        f32x8_t e8;
#pragma unroll
        for (int e = 0; e < 8; ++e) e8[e] = g[8 * c2 + e];
        const typename Ty<T>::frag fr = Ty<T>::cvt8(e8);
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = Ty<T>::mma(op(c2, db), fr, acc[db]);
      }
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const f32x4_t vv = op(q4, db);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db] = Ty<T>::mma(vv[e], g[4 * q4 + e], acc[db]);
        }
    }
  };

  const int y_end = ext;
  // The next block's rows are loaded into registers while the current block
  // is computed, with (K side) its queries' lse2 and D, (Q side) its keys'
  // score bias (0, or -inf for keys that take no part) and whether every
  // key of the block takes part.
  uint4 pf1[C::NPF], pf2[C::NPF];
  float pst0 = 0.f, pst1 = 0.f;
  bool pfull = true;
  auto fetch = [&](int yb) {
    if (!KSIDE) {
      load_rows<T, D>(pf1, Kg, p.ld_k, tok0, yb, ext, mrow, hoff, tid);
      load_rows<T, D>(pf2, Vg, p.ld_v, tok0, yb, ext, mrow, hoff, tid);
      const int y = yb + li;
      const bool ok = y < ext && (!mrow || mrow[y] != 0);
      pst0 = ok ? 0.f : kNegInf;
      pfull = __all(ok);
    } else {
      load_rows<T, D>(pf1, Qg, p.ld_q, tok0, yb, ext, mrow, hoff, tid);
      load_rows<T, D>(pf2, DOg, p.ld_do, tok0, yb, ext, mrow, hoff, tid);
      if (tid < C::BY) {
        const int y = yb + tid;
        const bool ok = y < ext && (!mrow || mrow[y] != 0);
        const float l = ok ? p.lse[(tok0 + y) * p.H + head] : kNegInf;
        pst0 = l == kNegInf ? kPosInf : l * l2e;
        pst1 = ok ? p.dsum[(tok0 + y) * p.H + head] : 0.f;
      }
    }
  };
  // the block at y0 into LDS (ystat: K side lse2 and D of its queries, Q
  // side its keys' bias), then the next block's loads go out; returns
  // whether every y of the block takes part (Q side)
  auto stage = [&](int y0) {
    if (!C::PREFETCH) fetch(y0);
    store_rows<T, D>(pf1, R1, tid);
    store_rows<T, D>(pf2, R2, tid);
    if (tid < C::BY) {
      ystat[tid] = pst0;
      ystat[C::BY + tid] = pst1;
    }
    const bool full = pfull;
    lds_barrier();
    if (C::PREFETCH && y0 + C::BY < y_end) fetch(y0 + C::BY);
    return full;
  };

  const unsigned char* r1_lane = R1 + (li * C::RPITCH + lh * C::HALF) * ES;
  const unsigned char* r2_lane = R2 + (li * C::RPITCH + lh * C::HALF) * ES;
  // the gradient products of a block from P (pm) and dS (ds)
  auto grads = [&](const f32x16_t& pm, const f32x16_t& ds) {
    if (!KSIDE) {
      grad_acc(acc1, top(R1), ds);             // dQ^T += K^T dS
    } else {
      grad_acc(acc1, top(R2), pm);             // dV^T += dO^T P
      grad_acc(acc2, top(R1), ds);             // dK^T += Q^T dS
    }
  };

  // Blocks where every pair of the wave lies beyond the band on one side:
  // one table row per term (E as the S accumulator's initial value, F in
  // the operand), no per-pair tests. Returns the block's sum of dS.
  auto far_block = [&](const uint4 (&xfr)[NU], bool full) {
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = e_far;
    s = mma_chain_lds<T, NU, NC>(r1_lane, xfr, s);
    const f32x16_t dp = mma_chain_lds<T, NU, NC>(r2_lane, xp, f32x16_t{});
    f32x16_t pm, ds;
    float fs = 0.f;
    if (!KSIDE) {
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] += ystat[rr_of(r) + 4 * lh];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c1, -lse2_x));
        pm[r] = pv;
        ds[r] = pv * (dp[r] - d_x);
        fs += ds[r];
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(ystat + 8 * g + 4 * lh);
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(ystat + C::BY + 8 * g + 4 * lh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], c1, -l4[e]));
          pm[r] = pv;
          ds[r] = pv * (dp[r] - d4[e]);
          fs += ds[r];
        }
      }
    }
    grads(pm, ds);
    return fs;
  };

  // The distance store is written in complete rows of the wave's 32 tokens.
  // With block n's dS in scratch row ri = 31 + (y - y0) - li, row ri holds
  // the distance u(ri) (Q side x0w - y0 + 31 - ri, K side y0 - x0w - 31 +
  // ri) for the tokens li in [31 - ri, 62 - ri]; the same distance is row
  // ri - 32 of block n+1. So rows 0..31 are complete after block n (tokens
  // li < 31 - ri came from block n-1 through `carry`), rows 32..62 wait for
  // block n+1 in `carry`, and after the wave's last band block they are
  // written with zeros for the tokens no block holds. Before the first band
  // block `carry` is zero. Rows at or beyond the band are not stored.
  float* carry = reinterpret_cast<float*>(smem + C::OFF_CARRY + wave * C::CARRY_BYTES);
  if (e_on)
    for (int x4 = lane; x4 < 31 * 8; x4 += 64)
      *reinterpret_cast<f32x4_t*>(carry + 4 * x4) = f32x4_t{0.f, 0.f, 0.f, 0.f};
  using DgE = typename std::conditional<ES == 2, uint16_t, float>::type;
  DgE* const dstore = reinterpret_cast<DgE*>(KSIDE ? p.dgk : p.dgq);
  const int64_t tw = tok0 + x0w;              // the wave's first token
  const bool al4 = (tw & 3) == 0;             // 4-token units start on 8-byte boundaries
  // the wave's tokens lie in groups tw/32 and tw/32 + 1: offsets from the first fit 32 bits
  DgE* const wbase = dstore + ((int64_t)head * p.dg_groups + (tw >> 5)) * p.dg_rows * 32;
  auto to_e = [](float v) -> DgE {
    if constexpr (ES == 2)
      return __builtin_bit_cast(
          uint16_t, (typename std::conditional<std::is_same<T, TF16>::value, _Float16, __bf16>::type)v);
    else
      return v;
  };
  auto put_rows = [&](int y0, bool upper) {
#pragma unroll 1
    for (int k = 0; k < 4; ++k) {
      const int j = lane + 64 * k;          // (row, 4-token unit)
      const int ri = (upper ? 32 : 0) + (j >> 3), c = j & 7;
      const int u = KSIDE ? y0 - x0w - 31 + ri : x0w - y0 + 31 - ri;
      if (ri > 62 || u <= -band || u >= band) continue;
      DgE v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int lt = 4 * c + e;
        const bool cur = upper ? (lt <= 62 - ri) : (lt >= 31 - ri);
        const float f = cur ? scr[ri * 32 + lt] : (upper ? 0.f : carry[ri * 32 + lt]);
        v[e] = to_e(f);
      }
      const int xl = x0w + 4 * c;           // unit-local first token of the unit
      const int tl = (int)(tw & 31) + 4 * c;  // token offset from the wave's first group
      DgE* dst = wbase + ((tl >> 5) * p.dg_rows + (u + p.dg_rb)) * 32 + (tl & 31);
      if (al4 && xl + 3 < len) {
        if constexpr (ES == 2)
          *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16),
                                                      (uint32_t)v[2] | ((uint32_t)v[3] << 16));
        else
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
      } else {
        // unaligned start or the unit's end: one element at a time (the
        // group of each token found separately)
        for (int e = 0; e < 4; ++e) {
          if (xl + e >= len) break;
          const int te = tl + e;
          wbase[((te >> 5) * p.dg_rows + (u + p.dg_rb)) * 32 + (te & 31)] = v[e];
        }
      }
    }
  };

  // Blocks with pairs inside the band (per wave: band products gathered
  // along the diagonal, dS stored by distance), or beyond it on both sides.
  auto general_block = [&](int y0) {
    const int vlo = x0w - (y0 + 31), vhi = x0w + 31 - y0;   // x - y over the wave's block
    const bool blk_far = terms && (vlo >= band || vhi <= -band);
    f32x16_t s;
    if (blk_far) {
      if (vhi <= -band && !far_lt_ready) {
        make_far(true);
        far_lt_ready = true;
      }
      uint4 xf[NU];
      lds_half_row<NU>(xf, xf_lds);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = e_far;
      s = mma_chain_lds<T, NU, NC>(r1_lane, xf, s);
    } else {
      s = mma_chain_lds<T, NU, NC>(r1_lane, xs, f32x16_t{});
      if (e_on) {
        // E[u][x] = ER[T(umin + u)] . xs_x over the 63 distances u = x - y
        const int umin = x0w - (y0 + 31);
#pragma unroll
        for (int ub = 0; ub < 2; ++ub) {
          uint4 rf[NU];
          load_half_row<NU>(rf, ERg + (int64_t)rel_row(p, umin + 32 * ub + li) * ld_rel_b);
          const f32x16_t e = mma_chain<T, NU, NC>(rf, xs, f32x16_t{});
#pragma unroll
          for (int r = 0; r < 16; ++r) scr[(ub * 32 + rr_of(r) + 4 * lh) * 32 + li] = e[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] += scr[(li - rr_of(r) - 4 * lh + 31) * 32 + li];
      }
      if (f_on) {
        // F[y][v] = R1_y . FR[T(vmin + v)] over the 63 distances v = y - x
        const int vmin = y0 - (x0w + 31);
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) {
          uint4 rf[NU];
          load_half_row<NU>(rf, FRg + (int64_t)rel_row(p, vmin + 32 * vb + li) * ld_rel_b);
          const f32x16_t f = mma_chain_lds<T, NU, NC>(r1_lane, rf, f32x16_t{});
#pragma unroll
          for (int r = 0; r < 16; ++r) scr[(rr_of(r) + 4 * lh) * 64 + vb * 32 + li] = f[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] += scr[(rr_of(r) + 4 * lh) * 65 + 31 - li];
      }
    }

    // P, dP, dS with every pair tested
    const f32x16_t dp = mma_chain_lds<T, NU, NC>(r2_lane, xp, f32x16_t{});
    f32x16_t pm, ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int yr = rr_of(r) + 4 * lh;
      const int y = y0 + yr;
      const bool y_valid = y < ext && (!mrow || mrow[y] != 0);
      const float lse_i = KSIDE ? ystat[yr] : lse2_x;
      const float d_i = KSIDE ? ystat[C::BY + yr] : d_x;
      const bool ok = x_valid && y_valid;
      const float pv = ok ? __builtin_amdgcn_exp2f(fmaf(s[r], c1, -lse_i)) : 0.f;
      pm[r] = pv;
      ds[r] = ok ? pv * (dp[r] - d_i) : 0.f;
    }
    grads(pm, ds);

    // pairs beyond the band: per-position sums; inside: the distance store
    // (selects, not branches: an if / else-if pair here became a private
    // two-element array indexed at run time, i.e. scratch-memory traffic)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int y = y0 + rr_of(r) + 4 * lh;
      const int u = KSIDE ? (y - x) : (x - y);   // query minus key
      far_gt += u >= band ? ds[r] : 0.f;
      far_lt += u <= -band ? ds[r] : 0.f;
    }
    if (e_on && !blk_far) {
      // dS of this wave's pairs into scratch row ri = 31 + (y - y0) - li,
      // whose distance (query minus key) does not depend on the lane; then
      // the rows complete after this block go to the store
#pragma unroll
      for (int r = 0; r < 16; ++r) scr[(31 + rr_of(r) + 4 * lh - li) * 32 + li] = ds[r];
      put_rows(y0, false);
      const int vlo_n = vlo - C::BY, vhi_n = vhi - C::BY;   // the next block's x - y range
      const bool next_band = y0 + C::BY < y_end && !(vlo_n >= band || vhi_n <= -band);
      if (next_band) {
        // rows 32..62 wait for the next block: carry row ri - 32
        for (int x4 = lane; x4 < 31 * 8; x4 += 64) {
          const int r = x4 >> 3, c4 = x4 & 7;
          *reinterpret_cast<f32x4_t*>(carry + r * 32 + 4 * c4) =
              *reinterpret_cast<const f32x4_t*>(scr + (32 + r) * 32 + 4 * c4);
        }
      } else {
        put_rows(y0, true);   // the wave's last band block: the rest of those rows is zero
      }
    }
  };

  // Block ranges: [0, n_gt) beyond the band below for every wave (u >= band
  // on the Q side), [n_lt, nb) beyond it above for every wave, the rest
  // general. Without position terms every block takes the plain path.
  const int nb = (y_end + C::BY - 1) / C::BY;
  int n_gt = nb, n_lt = nb;
  if (terms) {
    const int lim = x0 - 31 - band;                 // y0 <= lim: wave 0 (the closest) beyond the band
    n_gt = lim >= 0 ? min(nb, lim / C::BY + 1) : 0;
    const int lo = x0 + (C::BX - 1) + band;         // y0 >= lo: the last wave beyond the band
    n_lt = max(n_gt, min(nb, (lo + C::BY - 1) / C::BY));
  }
  if (C::PREFETCH) fetch(0);
  if (n_gt > 0) {
    uint4 xf[NU];
    if (terms) lds_half_row<NU>(xf, xf_lds);
    else {
#pragma unroll
      for (int u = 0; u < NU; ++u) xf[u] = xs[u];
    }
    float fs = 0.f;
    for (int n = 0; n < n_gt; ++n) {
      const bool full = stage(n * C::BY);
      fs += far_block(xf, full);
      lds_barrier();   // the block's LDS is rewritten next
    }
    // KSIDE: these blocks have y - x <= -band, i.e. query minus key <= -band
    if (KSIDE) far_lt += fs;
    else far_gt += fs;
  }
  for (int n = n_gt; n < n_lt; ++n) {
    stage(n * C::BY);
    general_block(n * C::BY);
    lds_barrier();   // the block's LDS is rewritten next; its stores may still be in flight
  }
  if (n_lt < nb) {
    if (!far_lt_ready) make_far(true);
    uint4 xf[NU];
    lds_half_row<NU>(xf, xf_lds);
    float fs = 0.f;
    for (int n = n_lt; n < nb; ++n) {
      const bool full = stage(n * C::BY);
      fs += far_block(xf, full);
      lds_barrier();
    }
    if (KSIDE) far_gt += fs;
    else far_lt += fs;
  }

  // rows of the distance store no band block of this wave covered
  if (dg_on && x0w < len) {
    // band blocks: y0 in (x0w - 31 - band, x0w + 31 + band), 0 <= y0 < ext
    int y_first = x0w - 31 - band < 0 ? 0 : ((x0w - 31 - band) / C::BY + 1) * C::BY;
    int y_last = min((nb - 1) * C::BY, ((x0w + 30 + band) / C::BY) * C::BY);
    int ulo = 1, uhi = 0;
    if (x0w < ext && y_first <= y_last) {
      ulo = KSIDE ? y_first - x0w - 31 : x0w - y_last - 31;
      uhi = KSIDE ? y_last - x0w + 31 : x0w - y_first + 31;
    }
    zero_rows(ulo, uhi);
  }

  // ---- epilogue --------------------------------------------------------------
  const float fgt = far_gt + __shfl_xor(far_gt, 32);   // both lane halves of position x
  const float flt = far_lt + __shfl_xor(far_lt, 32);
  if (!x_valid) {   // past the extent or masked: zero gradients
    write_zero_row();
    return;
  }
  if (lh == 0) {
    float* fs = KSIDE ? p.bfar : p.afar;
    fs[((tok0 + x) * p.H + head) * 2 + 0] = fgt;
    fs[((tok0 + x) * p.H + head) * 2 + 1] = flt;
  }
  float* part = KSIDE ? p.dk_part : p.dq_part;
  f32x16_t (&pacc)[NDB] = KSIDE ? acc2 : acc1;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dd = db * 32 + 8 * g + 4 * lh + e;
        part[((tok0 + x) * p.H + head) * D + dd] = tau * pacc[db][4 * g + e];
        if (KSIDE)
          from_f<T>(p.dv, (tok0 + x) * ((int64_t)p.H * D) + hoff + dd, acc1[db][4 * g + e]);
      }
}

// ---------------------------------------------------------------------------
// 4.-5. the distance sums as MFMA products
// ---------------------------------------------------------------------------

// MFMA operand of lane (n = lane % 32, reduction elements k0 + 8 (lane / 32)
// + 0..7 for 16-bit types, k0 + lane / 32 for fp32) from a row-major LDS
// block [k][n] with `pitch` elements per row: the transposing read
// ds_read_b64_tr_b16 for 16-bit types (two reads of four rows each).
template <class T>
__device__ __forceinline__ typename Ty<T>::frag kop_rows(const unsigned char* blk, int pitch, int k0,
                                                       int n0, int lane) {
  if constexpr (Ty<T>::ESIZE == 2) {
    const int g = lane >> 4, t = lane & 15;
    const unsigned char* a =
        blk + ((k0 + 8 * (g >> 1) + (t >> 2)) * pitch + n0 + 16 * (g & 1) + 4 * (t & 3)) * 2;
    const uint2 lo = lds_tr16(a), hi = lds_tr16(a + 4 * pitch * 2);
    return __builtin_bit_cast(typename Ty<T>::frag, make_uint4(lo.x, lo.y, hi.x, hi.y));
  } else {
    return reinterpret_cast<const float*>(blk)[(k0 + (lane >> 5)) * pitch + n0 + (lane & 31)];
  }
}

// MFMA operand of lane (m = lane % 32, the same reduction elements) from a
// row-major LDS block [m][k] (reduction index contiguous)
template <class T>
__device__ __forceinline__ typename Ty<T>::frag mop_rows(const unsigned char* blk, int pitch, int k0,
                                                       int m0, int lane) {
  if constexpr (Ty<T>::ESIZE == 2) {
    return __builtin_bit_cast(typename Ty<T>::frag,
                              ld16(blk + ((m0 + (lane & 31)) * pitch + k0 + 8 * (lane >> 5)) * 2));
  } else {
    return reinterpret_cast<const float*>(blk)[(m0 + (lane & 31)) * pitch + k0 + (lane >> 5)];
  }
}

// Position parts of dQ (C2P, KSIDE = false) and dK (P2C, KSIDE = true):
//   dq[t] = dq_part[t] + tau (sum_u Dq[u][t] kr[T(u)]
//                             + afar_gt[t] kr[top] + afar_lt[t] kr[bottom])
//   dk[t] = dk_part[t] + tau (sum_u Dk[u][t] qr[T(-u)]
//                             + bfar_gt[t] qr[bottom] + bfar_lt[t] qr[top])
// (u is query minus key; beyond the band C2P reads the top row for u >= band
// and the bottom row for u <= -band, P2C the other way round). As a product
// out^T [d x tokens] = R^T [d x U] D [U x tokens]: a workgroup owns 128
// tokens of one head (32 per wave) and walks the distances 32 at a time;
// the D block and the gathered table rows are staged row-major in LDS and
// both operands are read transposed. Every output row is rounded once.
template <class T, int D, bool KSIDE>
__global__ __launch_bounds__(256) void bwd_pos_grad_kernel(BwdParams p) {
  constexpr int ES = Ty<T>::ESIZE;
  constexpr int TB = 128, UB = 32, EPU = 16 / ES;
  constexpr int DP = TB + 32 / ES;     // D block pitch (elements): rows 32 bytes apart in the banks
  constexpr int RP = D + 32 / ES;      // table block pitch
  constexpr int NDB = D / 32;
  constexpr int KSTEP = ES == 2 ? 16 : 2;
  __shared__ __attribute__((aligned(16))) unsigned char dsb[UB * DP * ES];
  __shared__ __attribute__((aligned(16))) unsigned char rsb[UB * RP * ES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int head = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const bool on = KSIDE ? (p.flags & 2u) != 0 : (p.flags & 1u) != 0;
  const unsigned char* rel = reinterpret_cast<const unsigned char*>(KSIDE ? p.qr : p.kr);
  const unsigned char* dgs = reinterpret_cast<const unsigned char*>(KSIDE ? p.dgk : p.dgq);
  const int band = p.band;

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
  // D rows u0 .. u0+31 over tokens t0 .. t0+127 (four 32-token groups;
  // groups past the last token and rows past the band read as zero) and
  // the table rows these distances read, as 16-byte units: loaded into
  // registers one step ahead, stored to LDS when the step's turn comes
  constexpr int ND = (UB * (TB / EPU) + 255) / 256, NR = (UB * (D / EPU) + 255) / 256;
  uint4 pd[ND], pr[NR];
  auto fetch = [&](int u0) {
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      const int x = tid + 256 * k;
      const int r = x / (TB / EPU), c = x - r * (TB / EPU);
      const int u = u0 + r;
      const int64_t g = (t0 >> 5) + c / (32 / EPU);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (x < UB * (TB / EPU) && u < band && g < p.dg_groups)
        v = ld16(dgs + ((((int64_t)head * p.dg_groups + g) * p.dg_rows + (u + p.dg_rb)) * 32 +
                        EPU * (c % (32 / EPU))) * ES);
      pd[k] = v;
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int x = tid + 256 * k;
      const int r = x / (D / EPU), c = x - r * (D / EPU);
      const int u = u0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (x < UB * (D / EPU) && u < band)
        v = ld16(rel + ((int64_t)rel_row(p, KSIDE ? -u : u) * p.ld_rel + (int64_t)head * D + EPU * c) * ES);
      pr[k] = v;
    }
  };
  if (on) {
    fetch(-(band - 1));
    for (int u0 = -(band - 1); u0 < band; u0 += UB) {
#pragma unroll
      for (int k = 0; k < ND; ++k) {
        const int x = tid + 256 * k;
        const int r = x / (TB / EPU), c = x - r * (TB / EPU);
        if (x < UB * (TB / EPU)) *reinterpret_cast<uint4*>(dsb + (r * DP + EPU * c) * ES) = pd[k];
      }
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const int x = tid + 256 * k;
        const int r = x / (D / EPU), c = x - r * (D / EPU);
        if (x < UB * (D / EPU)) *reinterpret_cast<uint4*>(rsb + (r * RP + EPU * c) * ES) = pr[k];
      }
      lds_barrier();
      if (u0 + UB < band) fetch(u0 + UB);
#pragma unroll
      for (int k0 = 0; k0 < UB; k0 += KSTEP) {
        const auto bop = kop_rows<T>(dsb, DP, k0, 32 * wave, lane);
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = Ty<T>::mma(kop_rows<T>(rsb, RP, k0, 32 * db, lane), bop, acc[db]);
      }
      lds_barrier();
    }
  }
  const int64_t t = t0 + 32 * wave + li;
  if (t >= p.tokens) return;
  const float* part = KSIDE ? p.dk_part : p.dq_part;
  const float* fars = KSIDE ? p.bfar : p.afar;
  void* outp = KSIDE ? p.dk : p.dq;
  float fgt = 0.f, flt = 0.f;
  int r_gt = 0, r_lt = 0;
  if (on) {
    fgt = fars[(t * p.H + head) * 2 + 0];
    flt = fars[(t * p.H + head) * 2 + 1];
    const int row_top = rel_row(p, p.rel_max_len - 1), row_bot = rel_row(p, -(p.rel_max_len - 1));
    r_gt = KSIDE ? row_bot : row_top;
    r_lt = KSIDE ? row_top : row_bot;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = db * 32 + 8 * g + 4 * lh + e;
        float a = acc[db][4 * g + e];
        if (on) {
          a += fgt * to_f<T>(rel, (int64_t)r_gt * p.ld_rel + (int64_t)head * D + c);
          a += flt * to_f<T>(rel, (int64_t)r_lt * p.ld_rel + (int64_t)head * D + c);
        }
        from_f<T>(outp, t * ((int64_t)p.H * D) + (int64_t)head * D + c,
                  part[(t * p.H + head) * D + c] + p.tau * a);
      }
}

// W[h][b][u + band - 1] = sum over the tokens i of unit b of D[u][i] x_i
// (C2P: Dq with q; P2C: Dk with k), for |u| < band. As a product
// W [U x d] = D [U x tokens] X [tokens x d]: a workgroup owns 128 distances
// of one (unit, head) (32 per wave) and walks the unit's tokens 32 at a
// time from an 8-aligned start; X rows of tokens outside the unit are
// staged as zero, so the neighbouring units' entries of D add nothing.
template <class T, int D, bool KSIDE>
__global__ __launch_bounds__(256) void bwd_pos_w_kernel(BwdParams p) {
  constexpr int ES = Ty<T>::ESIZE;
  constexpr int UB = 128, IB = 32, EPU = 16 / ES;
  constexpr int DP = IB + 16 / ES;     // D block pitch (elements)
  constexpr int XP = D + 32 / ES;      // X block pitch
  constexpr int NDB = D / 32;
  constexpr int KSTEP = ES == 2 ? 16 : 2;
  __shared__ __attribute__((aligned(16))) unsigned char dsb[UB * DP * ES];
  __shared__ __attribute__((aligned(16))) unsigned char xsb[IB * XP * ES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int head = blockIdx.z, b = blockIdx.y;
  const bool on = KSIDE ? (p.flags & 2u) != 0 : (p.flags & 1u) != 0;
  if (!on) return;
  const int band = p.band;
  const int dg_rows = 2 * band - 1;
  const int wrows = 2 * band + 1;
  const int row0 = blockIdx.x * UB;
  const int len = unit_len(p, b);
  const int64_t tok0 = unit_base(p, b);
  const unsigned char* dgs = reinterpret_cast<const unsigned char*>(KSIDE ? p.dgk : p.dgq);
  const unsigned char* xg = reinterpret_cast<const unsigned char*>(KSIDE ? p.k : p.q);
  const int64_t ldx = KSIDE ? p.ld_k : p.ld_q;
  float* wout = KSIDE ? p.wk : p.wq;

  f32x16_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
  // token chunks are the 32-token groups of the store
  const int64_t ia = tok0 & ~(int64_t)31;
  for (int64_t i0 = ia; i0 < tok0 + len; i0 += IB) {
    const int64_t gbase = ((int64_t)head * p.dg_groups + (i0 >> 5)) * p.dg_rows;
    for (int x = tid; x < UB * (IB / EPU); x += 256) {
      const int r = x / (IB / EPU), c = x - r * (IB / EPU);
      const int row = row0 + r;   // distance row - (band - 1)
      // tokens of the group outside this sequence: their entries belong to
      // the neighbouring sequences or to no token, so they are masked here
      const int64_t i = i0 + EPU * c;
      const int lo = (int)max((int64_t)0, tok0 - i), hi = (int)min((int64_t)EPU, tok0 + len - i);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < dg_rows && lo < hi) {
        v = ld16(dgs + ((gbase + (row - (band - 1) + p.dg_rb)) * 32 + EPU * c) * ES);
        if (lo > 0 || hi < EPU) {
          uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < EPU; ++e) {
            if (e >= lo && e < hi) continue;
            if constexpr (ES == 2) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            else w[e] = 0u;
          }
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      *reinterpret_cast<uint4*>(dsb + (r * DP + EPU * c) * ES) = v;
    }
    for (int x = tid; x < IB * (D / EPU); x += 256) {
      const int r = x / (D / EPU), c = x - r * (D / EPU);
      const int64_t i = i0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (i >= tok0 && i < tok0 + len) v = ld16(xg + (i * ldx + (int64_t)head * D + EPU * c) * ES);
      *reinterpret_cast<uint4*>(xsb + (r * XP + EPU * c) * ES) = v;
    }
    __syncthreads();
#pragma unroll
    for (int k0 = 0; k0 < IB; k0 += KSTEP) {
      const auto aop = mop_rows<T>(dsb, DP, k0, 32 * wave, lane);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = Ty<T>::mma(aop, kop_rows<T>(xsb, XP, k0, 32 * db, lane), acc[db]);
    }
    __syncthreads();
  }
  // lane: column c = 32 db + li; registers: rows 8 g + 4 lh + e of the wave's 32
  const int64_t wbase = ((int64_t)head * p.units + b) * wrows * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = row0 + 32 * wave + 8 * g + 4 * lh + e;
        if (row < dg_rows) wout[wbase + (int64_t)row * D + 32 * db + li] = acc[db][4 * g + e];
      }
}

// the two rows of W past the distances: sum over the unit's tokens of the
// beyond-band sums (u >= band, then u <= -band) times q (C2P) and k (P2C).
// One workgroup per (unit, head): a thread owns one 16-byte column group
// and a strided subset of the tokens; the token groups are then added in a
// fixed order.
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pos_farw_kernel(BwdParams p) {
  constexpr int ES = Ty<T>::ESIZE, EPU = 16 / ES;
  constexpr int CG = D / EPU, TG = 256 / CG;
  const int head = blockIdx.y, b = blockIdx.x;
  const int len = unit_len(p, b);
  const int64_t tok0 = unit_base(p, b);
  const int band = p.band;
  const int wrows = 2 * band + 1;
  const bool c2p = (p.flags & 1u) != 0, p2c = (p.flags & 2u) != 0;
  const int cg = threadIdx.x % CG, tg = threadIdx.x / CG;
  const unsigned char* qb = reinterpret_cast<const unsigned char*>(p.q);
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(p.k);
  float s[4][EPU];   // q * afar_gt, q * afar_lt, k * bfar_gt, k * bfar_lt
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int e = 0; e < EPU; ++e) s[w][e] = 0.f;
  auto unpack = [](uint4 u, float (&f)[EPU]) {
    if constexpr (ES == 2) {
      const auto v = __builtin_bit_cast(typename Ty<T>::frag, u);
#pragma unroll
      for (int e = 0; e < EPU; ++e) f[e] = (float)v[e];
    } else {
      const f32x4_t v = __builtin_bit_cast(f32x4_t, u);
#pragma unroll
      for (int e = 0; e < EPU; ++e) f[e] = v[e];
    }
  };
#pragma unroll 2
  for (int i = tg; i < len; i += TG) {
    const int64_t t = tok0 + i;
    float f[EPU];
    if (c2p) {
      unpack(ld16(qb + (t * p.ld_q + (int64_t)head * D + EPU * cg) * ES), f);
      const float a0 = p.afar[(t * p.H + head) * 2 + 0], a1 = p.afar[(t * p.H + head) * 2 + 1];
#pragma unroll
      for (int e = 0; e < EPU; ++e) { s[0][e] += a0 * f[e]; s[1][e] += a1 * f[e]; }
    }
    if (p2c) {
      unpack(ld16(kb + (t * p.ld_k + (int64_t)head * D + EPU * cg) * ES), f);
      const float b0 = p.bfar[(t * p.H + head) * 2 + 0], b1 = p.bfar[(t * p.H + head) * 2 + 1];
#pragma unroll
      for (int e = 0; e < EPU; ++e) { s[2][e] += b0 * f[e]; s[3][e] += b1 * f[e]; }
    }
  }
  __shared__ float red[TG][4 * D];
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int e = 0; e < EPU; ++e) red[tg][w * D + EPU * cg + e] = s[w][e];
  __syncthreads();
  const int64_t wbase = ((int64_t)head * p.units + b) * wrows * D;
  for (int c = threadIdx.x; c < 4 * D; c += 256) {
    float r = 0.f;
    for (int g = 0; g < TG; ++g) r += red[g][c];
    const int w = c / D, col = c - w * D;
    float* dst = w < 2 ? p.wq : p.wk;
    dst[wbase + (int64_t)(2 * band - 1 + (w & 1)) * D + col] = r;
  }
}

// ---------------------------------------------------------------------------
// 6. dkr / dqr rows: sequences in order, then the distances of each row
// ---------------------------------------------------------------------------

// first distance u in [lo, hi) with T(u) >= r (hi if none); T is non-decreasing
__device__ int first_dist_at_least(const BwdParams& p, int lo, int hi, int r) {
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (rel_row(p, mid) >= r) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

template <class T>
__global__ __launch_bounds__(256) void bwd_pos_rel_kernel(BwdParams p, int d) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t HD = (int64_t)p.H * d;
  if (w >= (int64_t)p.n_rel * HD) return;
  const int r = (int)(w / HD);
  const int c = (int)(w - (int64_t)r * HD);
  const int head = c / d, e = c - head * d;
  const int band = p.band;
  const int64_t wrows = 2 * (int64_t)band + 1;
  const int row_top = rel_row(p, p.rel_max_len - 1);
  const int row_bot = rel_row(p, -(p.rel_max_len - 1));
  // distances inside the band whose row is r: C2P reads T(u), P2C T(-u)
  const int ua = first_dist_at_least(p, -(band - 1), band, r);
  const int ub = first_dist_at_least(p, -(band - 1), band, r + 1);   // C2P: u in [ua, ub)
  // P2C: T(-u) = r  <=>  -u in [ua, ub)  <=>  u in (-ub, -ua]
  float skr = 0.f, sqr = 0.f;
  for (int b = 0; b < p.units; ++b) {
    const int64_t wbase = ((int64_t)head * p.units + b) * wrows * d + e;
    if (p.flags & 1u)
      for (int u = ua; u < ub; ++u) skr += p.wq[wbase + (int64_t)(u + band - 1) * d];
    if (p.flags & 2u)
      for (int u = -ub + 1; u <= -ua; ++u)
        if (u > -band && u < band) sqr += p.wk[wbase + (int64_t)(u + band - 1) * d];
    const int64_t fgt = wbase + (int64_t)(2 * band - 1) * d, flt = fgt + d;
    if (p.flags & 1u) {
      if (r == row_top) skr += p.wq[fgt];
      if (r == row_bot) skr += p.wq[flt];
    }
    if (p.flags & 2u) {
      if (r == row_bot) sqr += p.wk[fgt];
      if (r == row_top) sqr += p.wk[flt];
    }
  }
  if (p.dkr) from_f<T>(p.dkr, w, p.tau * skr);
  if (p.dqr) from_f<T>(p.dqr, w, p.tau * sqr);
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

template <class T, int D>
int launch_t_d(BwdParams& p, bool varlen, hipStream_t stream) {
  typedef BCfg<T, D> C;
  int64_t n_work;
  if (!varlen) {
    p.n_qtiles = (p.L + C::BX - 1) / C::BX;
    n_work = (int64_t)p.B * p.H * p.n_qtiles;
  } else {
    p.n_qtiles = (int32_t)(p.tokens / C::BX + p.nseq);
    n_work = (int64_t)p.H * p.n_qtiles;
  }
  if (n_work <= 0) return 0;
  if (n_work > 0x7fffffffLL) return 2;
  p.n_work = (int32_t)n_work;
  const dim3 grid((unsigned)n_work), block(C::NT);
  if (varlen) {
    hipLaunchKernelGGL((bwd_main_kernel<T, D, false, true>), grid, block, 0, stream, p);
    hipLaunchKernelGGL((bwd_main_kernel<T, D, true, true>), grid, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL((bwd_main_kernel<T, D, false, false>), grid, block, 0, stream, p);
    hipLaunchKernelGGL((bwd_main_kernel<T, D, true, false>), grid, block, 0, stream, p);
  }
  const dim3 gg((unsigned)((p.tokens + 127) / 128), (unsigned)p.H);
  hipLaunchKernelGGL((bwd_pos_grad_kernel<T, D, false>), gg, dim3(256), 0, stream, p);
  hipLaunchKernelGGL((bwd_pos_grad_kernel<T, D, true>), gg, dim3(256), 0, stream, p);
  if (p.flags) {   // dkr / dqr exist only with a position term
    const dim3 gw((unsigned)((2 * p.band - 1 + 127) / 128), (unsigned)p.units, (unsigned)p.H);
    hipLaunchKernelGGL((bwd_pos_w_kernel<T, D, false>), gw, dim3(256), 0, stream, p);
    hipLaunchKernelGGL((bwd_pos_w_kernel<T, D, true>), gw, dim3(256), 0, stream, p);
    hipLaunchKernelGGL((bwd_pos_farw_kernel<T, D>), dim3((unsigned)p.units, (unsigned)p.H), dim3(256), 0, stream,
                       p);
    const int64_t rcells = (int64_t)p.n_rel * p.H * D;
    hipLaunchKernelGGL(bwd_pos_rel_kernel<T>, dim3((unsigned)((rcells + 255) / 256)), dim3(256), 0, stream, p,
                       D);
  }
  return 0;
}

template <class T>
int launch_bwd_t(BwdParams& p, int d, bool varlen, hipStream_t stream) {
  const int64_t rows = p.tokens * p.H;
  hipLaunchKernelGGL(bwd_dsum_kernel<T>, dim3((unsigned)min((rows + 255) / 256 + 1, (int64_t)16384)), dim3(256),
                     0, stream, p, d);
  switch (d) {
    case 32: return launch_t_d<T, 32>(p, varlen, stream);
    case 64: return launch_t_d<T, 64>(p, varlen, stream);
    case 128: return launch_t_d<T, 128>(p, varlen, stream);
    default: return 2;
  }
}

}  // namespace

namespace {
// rows of a distance-store group: dg_rb odd and >= band - 1, then band more
// rows, rounded up to even
int32_t dg_rb_of(int32_t band) { return (band - 1) | 1; }
int32_t dg_rows_of(int32_t band) { return (dg_rb_of(band) + band + 1) & ~1; }
}  // namespace

int64_t bwd_workspace_bytes(int64_t tokens, int32_t units, int32_t H, int32_t d, int esize,
                            int32_t band) {
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t th = tokens * H;
  const int64_t wrows = 2 * (int64_t)band + 1;
  const int64_t dg_bytes = al((int64_t)H * ((tokens + 31) / 32) * dg_rows_of(band) * 32 * esize);
  return al(th * 4) + 2 * al(th * d * 4) + 2 * al(th * 2 * 4) + 2 * dg_bytes +
         2 * al((int64_t)H * units * wrows * d * 4);
}

void bwd_carve_workspace(BwdParams& p, void* ws, int d, int esize) {
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  unsigned char* w = reinterpret_cast<unsigned char*>(ws);
  const int64_t th = p.tokens * p.H;
  const int64_t wrows = 2 * (int64_t)p.band + 1;
  p.dg_groups = (p.tokens + 31) / 32;
  p.dg_rb = dg_rb_of(p.band);
  p.dg_rows = dg_rows_of(p.band);
  const int64_t dg_bytes = al((int64_t)p.H * p.dg_groups * p.dg_rows * 32 * esize);
  p.dsum = reinterpret_cast<float*>(w); w += al(th * 4);
  p.dq_part = reinterpret_cast<float*>(w); w += al(th * d * 4);
  p.dk_part = reinterpret_cast<float*>(w); w += al(th * d * 4);
  p.afar = reinterpret_cast<float*>(w); w += al(th * 2 * 4);
  p.bfar = reinterpret_cast<float*>(w); w += al(th * 2 * 4);
  p.dgq = w; w += dg_bytes;
  p.dgk = w; w += dg_bytes;
  p.wq = reinterpret_cast<float*>(w); w += al((int64_t)p.H * p.units * wrows * d * 4);
  p.wk = reinterpret_cast<float*>(w);
}

int launch_bwd(BwdParams& p, int dtype, int d, bool varlen, hipStream_t stream) {
  int st;
  switch (dtype) {
    case 0: st = launch_bwd_t<TF32>(p, d, varlen, stream); break;
    case 1: st = launch_bwd_t<TF16>(p, d, varlen, stream); break;
    case 2: st = launch_bwd_t<TBF16>(p, d, varlen, stream); break;
    default: return 2;
  }
  if (st) return st;
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace dattn
