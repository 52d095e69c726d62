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
//     terms, as the forward's band path: per wave E = kr-row x q and
//     F = k x qr-row products gathered along the diagonal through LDS), P
//     and dS, accumulates the content part of dQ (dS K) and, per query,
//     the sums of dS over the pairs whose distance u = i - j lies beyond
//     the band (|u| >= band, where the table is constant); the dS of pairs
//     inside the band are stored by distance, Dg[h][u][query token].
//  3. main<K side>: a workgroup owns 128 keys and walks the queries. The
//     score is symmetric under exchanging (q, kr) with (k, qr) and i with j,
//     so the same tile routine with those operands exchanged yields S in
//     the key-major layout; it accumulates dV, the content part of dK and
//     the per-key sums beyond the band.
//  4. pos_dq / pos_dk: the position parts of dQ and dK from Dg (a
//     distance-indexed product with the table rows) and the sums beyond
//     the band (the table's end rows); each output row is rounded once.
//  5. pos_w: per (sequence, head) and distance, W_u = sum_i Dg[u][i] q_i
//     and sum_j Dg[u][j+u] k_j, plus the beyond-band sums times q or k.
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
  static constexpr int TPITCH = ES == 2 ? BY + 8 : BY + 4;   // transposed block pitch
  static constexpr int ROWS_BYTES = BY * RPITCH * ES;
  static constexpr int TR_BYTES = (D * TPITCH * ES + 15) / 16 * 16;
  static constexpr int SCR_BYTES = 64 * 32 * 4;      // per wave: 64 distances x 32 positions
  // LDS: two row blocks, two transposed blocks, per-wave scratch, per-y stats
  static constexpr int OFF_R1 = 0;
  static constexpr int OFF_R2 = OFF_R1 + ROWS_BYTES;
  static constexpr int OFF_T1 = OFF_R2 + ROWS_BYTES;
  static constexpr int OFF_T2 = OFF_T1 + TR_BYTES;
  static constexpr int OFF_SCR = OFF_T2 + TR_BYTES;
  static constexpr int OFF_STAT = OFF_SCR + NW * SCR_BYTES;
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
// 1. D_i = dO_i . O_i; also clears the distance-indexed dS store
// ---------------------------------------------------------------------------

template <class T>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(BwdParams p, int d) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t rows = p.tokens * p.H;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < rows; idx += stride) {
    const int64_t t = idx / p.H;
    const int h = (int)(idx - t * p.H);
    float acc = 0.f;
    for (int e = 0; e < d; ++e)
      acc += to_f<T>(p.dout, t * p.ld_do + (int64_t)h * d + e) * to_f<T>(p.o, t * p.ld_o + (int64_t)h * d + e);
    p.dsum[idx] = acc;
  }
  // zero Dg: entries of pairs outside every sequence are never written
  const int64_t n_dg = (int64_t)p.H * (2 * p.band - 1) * p.tokens;
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n_dg; x += stride) from_f<T>(p.dg, x, 0.f);
}

// ---------------------------------------------------------------------------
// 2./3. the tile loops
// ---------------------------------------------------------------------------

// Stage a block of BY rows (positions y0..y0+BY-1 of the unit, rows past
// len are zero) into LDS: row-major (pitch RPITCH) and, optionally, the
// transpose [D][BY] in the MFMA operand order of the forward's V^T.
template <class T, int D>
__device__ __forceinline__ void stage_rows(const unsigned char* g, int64_t ld, int64_t tok0, int y0,
                                           int ext, const uint8_t* mrow, int64_t hoff,
                                           unsigned char* rows, unsigned char* tr, int tid) {
  typedef BCfg<T, D> C;
  constexpr int ES = C::ES;
  constexpr int JOBS = (C::BY / 2) * C::UPR;   // (row pair, unit)
  for (int x = tid; x < JOBS; x += C::NT) {
    const int pr = x / C::UPR, u = x - pr * C::UPR;
    uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
    const int ya = y0 + 2 * pr, yb = ya + 1;
    // rows of positions that take no part (past the extent, masked) are zero
    if (ya < ext && (!mrow || mrow[ya])) a = ld16(g + ((tok0 + ya) * ld + hoff) * ES + 16 * u);
    if (yb < ext && (!mrow || mrow[yb])) b = ld16(g + ((tok0 + yb) * ld + hoff) * ES + 16 * u);
    *reinterpret_cast<uint4*>(rows + ((2 * pr) * C::RPITCH) * ES + 16 * u) = a;
    *reinterpret_cast<uint4*>(rows + ((2 * pr + 1) * C::RPITCH) * ES + 16 * u) = b;
    if (tr) {
      const uint32_t a4[4] = {a.x, a.y, a.z, a.w}, b4[4] = {b.x, b.y, b.z, b.w};
      if constexpr (ES == 2) {
        uint32_t* t32 = reinterpret_cast<uint32_t*>(tr);
        const int pp = v_pos(2 * pr) >> 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          t32[(((8 * u + e) * C::TPITCH) >> 1) + pp] = __builtin_amdgcn_perm(b4[e >> 1], a4[e >> 1], sel);
        }
      } else {
        uint2* t64 = reinterpret_cast<uint2*>(tr);
#pragma unroll
        for (int e = 0; e < 4; ++e) t64[((4 * u + e) * C::TPITCH + 2 * pr) >> 1] = make_uint2(a4[e], b4[e]);
      }
    }
  }
}

// KSIDE = false: lanes own queries (x = i), the loop walks keys (y = j).
// KSIDE = true:  lanes own keys (x = j), the loop walks queries (y = i).
template <class T, int D, bool KSIDE, bool VARLEN>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdParams p) {
  typedef BCfg<T, D> C;
  constexpr int ES = C::ES;
  constexpr int NU = C::NU;
  constexpr int NC = C::NC;
  constexpr int NDB = C::NDB;
  constexpr int NT = C::NT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
  unsigned char* R1 = smem + C::OFF_R1;   // rows for S: keys (Q side) / queries (K side)
  unsigned char* R2 = smem + C::OFF_R2;   // rows for dP: V (Q side) / dO (K side)
  unsigned char* T1 = smem + C::OFF_T1;   // K^T (Q side) / dO^T (K side)
  unsigned char* T2 = smem + C::OFF_T2;   // Q^T (K side)
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
  const float l2e = 1.4426950408889634f;
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
  if (x0 >= ext) {   // uniform: no position of this tile takes part
    write_zero_row();
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
  // Q side: this query's log-sum-exp and D
  float lse_x = kNegInf, d_x = 0.f;
  if (!KSIDE && x_valid) {
    lse_x = p.lse[(tok0 + x) * p.H + head];
    d_x = p.dsum[(tok0 + x) * p.H + head];
  }

  f32x16_t acc1[NDB], acc2[NDB];   // Q side: dQ^T; K side: dV^T (acc1), dK^T (acc2)
#pragma unroll
  for (int db = 0; db < NDB; ++db) { acc1[db] = f32x16_t{}; acc2[db] = f32x16_t{}; }
  float far_gt = 0.f, far_lt = 0.f;   // sums of dS over pairs with u >= band / u <= -band
  const int band = p.band;

  constexpr int V_LANE = ES == 2 ? 8 : 4;
  const unsigned char* t1_base = T1 + (li * C::TPITCH + V_LANE * lh) * ES;
  const unsigned char* t2_base = T2 + (li * C::TPITCH + V_LANE * lh) * ES;
  auto top = [](const unsigned char* base) {
    return [=](int c, int db) {
      if constexpr (ES == 2)
        return __builtin_bit_cast(typename Ty<T>::frag, ld16(base + (db * 32 * C::TPITCH + 16 * c) * ES));
      else
        return *reinterpret_cast<const f32x4_t*>(base + (db * 32 * C::TPITCH + 8 * c) * ES);
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

  const int64_t dg_rows = 2 * (int64_t)band - 1;
  const int y_end = ext;
  for (int y0 = 0; y0 < y_end; y0 += C::BY) {
    // ---- stage the block's rows ----------------------------------------------
    if (!KSIDE) {
      stage_rows<T, D>(Kg, p.ld_k, tok0, y0, ext, mrow, hoff, R1, T1, tid);
      stage_rows<T, D>(Vg, p.ld_v, tok0, y0, ext, mrow, hoff, R2, nullptr, tid);
    } else {
      stage_rows<T, D>(Qg, p.ld_q, tok0, y0, ext, mrow, hoff, R1, T2, tid);
      stage_rows<T, D>(DOg, p.ld_do, tok0, y0, ext, mrow, hoff, R2, T1, tid);
      if (tid < C::BY) {
        const int y = y0 + tid;
        const bool ok = y < ext && (!mrow || mrow[y] != 0);
        ystat[tid] = ok ? p.lse[(tok0 + y) * p.H + head] : kNegInf;
        ystat[C::BY + tid] = ok ? p.dsum[(tok0 + y) * p.H + head] : 0.f;
      }
    }
    __syncthreads();

    // ---- scores of the block: lanes x, registers y ---------------------------
    const unsigned char* r1_lane = R1 + (li * C::RPITCH + lh * C::HALF) * ES;
    f32x16_t s = mma_chain_lds<T, NU, NC>(r1_lane, xs, f32x16_t{});
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

    // ---- P, dP, dS -------------------------------------------------------------
    const unsigned char* r2_lane = R2 + (li * C::RPITCH + lh * C::HALF) * ES;
    const f32x16_t dp = mma_chain_lds<T, NU, NC>(r2_lane, xp, f32x16_t{});
    f32x16_t pm, ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int yr = rr_of(r) + 4 * lh;
      const int y = y0 + yr;
      const bool y_valid = y < ext && (!mrow || mrow[y] != 0);
      float lse_i, d_i;
      if (!KSIDE) { lse_i = lse_x; d_i = d_x; }
      else { lse_i = ystat[yr]; d_i = ystat[C::BY + yr]; }
      const bool ok = x_valid && y_valid && lse_i != kNegInf;
      const float pv = ok ? __builtin_amdgcn_exp2f((s[r] * tau - lse_i) * l2e) : 0.f;
      pm[r] = pv;
      ds[r] = ok ? pv * (dp[r] - d_i) : 0.f;
    }

    // ---- gradient products -----------------------------------------------------
    if (!KSIDE) {
      grad_acc(acc1, top(t1_base), ds);        // dQ^T += K^T dS
    } else {
      grad_acc(acc1, top(t1_base), pm);        // dV^T += dO^T P
      grad_acc(acc2, top(t2_base), ds);        // dK^T += Q^T dS
    }

    // ---- pairs beyond the band: per-position sums; inside (Q side): Dg --------
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int y = y0 + rr_of(r) + 4 * lh;
      const int u = KSIDE ? (y - x) : (x - y);   // query minus key
      if (u >= band) far_gt += ds[r];
      else if (u <= -band) far_lt += ds[r];
    }
    if (!KSIDE) {
      // dS of this wave's pairs by distance u = x - y: scratch [u - umin][x]
      const int umin = x0w - (y0 + 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) scr[(li - rr_of(r) - 4 * lh + 31) * 32 + li] = ds[r];
      // rows u of Dg hold consecutive query tokens: lanes 0-31 write row
      // 2k, lanes 32-63 row 2k+1
      for (int k2 = 0; k2 < 32; ++k2) {
        const int ui = 2 * k2 + lh;
        const int u = umin + ui;
        const int y = x - u;
        if (ui < 63 && u > -band && u < band && x_in && y >= y0 && y < y0 + C::BY && y < ext) {
          const int64_t idx = ((int64_t)head * dg_rows + (u + band - 1)) * p.tokens + tok0 + x;
          from_f<T>(p.dg, idx, scr[ui * 32 + li]);
        }
      }
    }
    __syncthreads();   // the block's LDS is rewritten next
  }

  // ---- epilogue --------------------------------------------------------------
  const float fgt = far_gt + __shfl_xor(far_gt, 32);   // both lane halves of position x
  const float flt = far_lt + __shfl_xor(far_lt, 32);
  if (!x_in) {
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
// 4. position parts of dQ (C2P) and dK (P2C); every row rounded once
// ---------------------------------------------------------------------------

// KSIDE = false: dq[t] = dq_part[t] + tau (sum_u Dg[u][t] kr[T(u)]
//                          + afar_gt[t] kr[top] + afar_lt[t] kr[bottom])
// KSIDE = true:  dk[t] = dk_part[t] + tau (sum_u Dg[u][t+u] qr[T(-u)]
//                          + bfar_gt[t] qr[bottom] + bfar_lt[t] qr[top])
// (beyond the band C2P reads the top row for u >= band and the bottom row
// for u <= -band; P2C, which reads T(-u), the other way round.)
// One workgroup per (32 tokens, head); distances in chunks of 64 through LDS.
template <class T, bool KSIDE>
__global__ __launch_bounds__(256) void bwd_pos_grad_kernel(BwdParams p, int d) {
  constexpr int TB = 32, UB = 64;
  const int head = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const bool on = KSIDE ? (p.flags & 2u) != 0 : (p.flags & 1u) != 0;
  const void* rel = KSIDE ? p.qr : p.kr;
  const float* part = KSIDE ? p.dk_part : p.dq_part;
  const float* fars = KSIDE ? p.bfar : p.afar;
  void* outp = KSIDE ? p.dk : p.dq;
  const int band = p.band;
  const int64_t dg_rows = 2 * (int64_t)band - 1;
  __shared__ float dgs[UB][TB + 1];
  __shared__ float rrow[UB][128 + 1];
  // this thread's outputs: column c, tokens tg, tg + per, ...
  const int c = threadIdx.x % d;
  const int per = 256 / d;                 // token groups
  const int tg = threadIdx.x / d;
  constexpr int MAXK = TB / 2;             // d >= 32: at most 16 tokens per thread
  const int nk = TB / per;
  float acc[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) acc[k] = 0.f;
  if (on) {
    for (int u0 = -(band - 1); u0 < band; u0 += UB) {
      __syncthreads();
      for (int x = threadIdx.x; x < UB * TB; x += 256) {
        const int ui = x / TB, tt = x - ui * TB;
        const int u = u0 + ui;
        float val = 0.f;
        const int64_t col = t0 + tt + (KSIDE ? u : 0);
        if (u < band && t0 + tt < p.tokens && col >= 0 && col < p.tokens)
          val = to_f<T>(p.dg, ((int64_t)head * dg_rows + (u + band - 1)) * p.tokens + col);
        dgs[ui][tt] = val;
      }
      for (int x = threadIdx.x; x < UB * d; x += 256) {
        const int ui = x / d, e = x - ui * d;
        const int u = u0 + ui;
        rrow[ui][e] = u < band ? to_f<T>(rel, (int64_t)rel_row(p, KSIDE ? -u : u) * p.ld_rel + (int64_t)head * d + e)
                               : 0.f;
      }
      __syncthreads();
      const int nu = min(UB, band - u0);
      for (int ui = 0; ui < nu; ++ui) {
        const float rv = rrow[ui][c];
#pragma unroll
        for (int k = 0; k < MAXK; ++k)
          if (k < nk) acc[k] += dgs[ui][tg + k * per] * rv;
      }
    }
  }
  const int row_top = on ? rel_row(p, p.rel_max_len - 1) : 0;
  const int row_bot = on ? rel_row(p, -(p.rel_max_len - 1)) : 0;
  const int r_gt = KSIDE ? row_bot : row_top, r_lt = KSIDE ? row_top : row_bot;
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    const int64_t t = t0 + tg + k * per;
    if (k >= nk || t >= p.tokens) continue;
    float a = acc[k];
    if (on) {
      a += fars[(t * p.H + head) * 2 + 0] * to_f<T>(rel, (int64_t)r_gt * p.ld_rel + (int64_t)head * d + c);
      a += fars[(t * p.H + head) * 2 + 1] * to_f<T>(rel, (int64_t)r_lt * p.ld_rel + (int64_t)head * d + c);
    }
    from_f<T>(outp, t * ((int64_t)p.H * d) + (int64_t)head * d + c,
              part[(t * p.H + head) * d + c] + p.tau * a);
  }
}

// ---------------------------------------------------------------------------
// 5. per (head, unit): W_u = sum_i Dg[u][i] q_i (C2P) and sum_j Dg[u][j+u] k_j
//    (P2C) for |u| < band; then the beyond-band sums times q and k
// ---------------------------------------------------------------------------

// Rows of W: 0 .. 2band-2 are the distances u = row - (band-1); row 2band-1
// holds the u >= band sums, row 2band the u <= -band sums. One workgroup per
// (64 rows, unit, head); positions in chunks of 32 through LDS.
template <class T>
__global__ __launch_bounds__(256) void bwd_pos_w_kernel(BwdParams p, int d) {
  constexpr int RB = 64, IB = 32;
  const int head = blockIdx.z, b = blockIdx.y;
  const int band = p.band;
  const int dg_rows = 2 * band - 1;
  const int wrows = 2 * band + 1;
  const int row0 = blockIdx.x * RB;
  const int len = unit_len(p, b);
  const int64_t tok0 = unit_base(p, b);
  const int64_t wbase = ((int64_t)head * p.units + b) * wrows * d;
  const bool c2p = (p.flags & 1u) != 0, p2c = (p.flags & 2u) != 0;
  __shared__ float aq[RB][IB + 1], ak[RB][IB + 1];
  __shared__ float qs[IB][128 + 1], ks[IB][128 + 1];
  const int c = threadIdx.x % d;
  const int per = 256 / d;
  const int rg = threadIdx.x / d;
  constexpr int MAXR = RB / 2;   // d >= 32: at most 32 rows per thread
  const int nr = RB / per;
  float oq[MAXR], ok[MAXR];
#pragma unroll
  for (int k = 0; k < MAXR; ++k) { oq[k] = 0.f; ok[k] = 0.f; }
  for (int i0 = 0; i0 < len; i0 += IB) {
    __syncthreads();
    for (int x = threadIdx.x; x < RB * IB; x += 256) {
      const int rl = x / IB, il = x - rl * IB;
      const int row = row0 + rl, i = i0 + il;
      float vq = 0.f, vk = 0.f;
      if (row < wrows && i < len) {
        if (row < dg_rows) {
          const int u = row - (band - 1);
          const int64_t drow = ((int64_t)head * dg_rows + row) * p.tokens + tok0;
          // pair (i, i - u) for q; pair (i + u, i) for k (i is then the key)
          if (c2p && i - u >= 0 && i - u < len) vq = to_f<T>(p.dg, drow + i);
          if (p2c && i + u >= 0 && i + u < len) vk = to_f<T>(p.dg, drow + i + u);
        } else {
          const int which = row - dg_rows;
          if (c2p) vq = p.afar[((tok0 + i) * p.H + head) * 2 + which];
          if (p2c) vk = p.bfar[((tok0 + i) * p.H + head) * 2 + which];
        }
      }
      aq[rl][il] = vq;
      ak[rl][il] = vk;
    }
    for (int x = threadIdx.x; x < IB * d; x += 256) {
      const int il = x / d, e = x - il * d;
      const int i = i0 + il;
      const bool in = i < len;
      qs[il][e] = (c2p && in) ? to_f<T>(p.q, (tok0 + i) * p.ld_q + (int64_t)head * d + e) : 0.f;
      ks[il][e] = (p2c && in) ? to_f<T>(p.k, (tok0 + i) * p.ld_k + (int64_t)head * d + e) : 0.f;
    }
    __syncthreads();
    for (int il = 0; il < IB; ++il) {
      const float qv = qs[il][c], kv = ks[il][c];
#pragma unroll
      for (int k = 0; k < MAXR; ++k)
        if (k < nr) {
          oq[k] += aq[rg + k * per][il] * qv;
          ok[k] += ak[rg + k * per][il] * kv;
        }
    }
  }
#pragma unroll
  for (int k = 0; k < MAXR; ++k) {
    const int row = row0 + rg + k * per;
    if (k >= nr || row >= wrows) continue;
    p.wq[wbase + (int64_t)row * d + c] = oq[k];
    p.wk[wbase + (int64_t)row * d + c] = ok[k];
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
int launch_main(BwdParams& p, bool varlen, hipStream_t stream) {
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
  return 0;
}

template <class T>
int launch_bwd_t(BwdParams& p, int d, bool varlen, hipStream_t stream) {
  const int64_t rows = p.tokens * p.H;
  hipLaunchKernelGGL(bwd_dsum_kernel<T>, dim3((unsigned)min((rows + 255) / 256 + 1, (int64_t)16384)), dim3(256),
                     0, stream, p, d);
  int st;
  switch (d) {
    case 32: st = launch_main<T, 32>(p, varlen, stream); break;
    case 64: st = launch_main<T, 64>(p, varlen, stream); break;
    case 128: st = launch_main<T, 128>(p, varlen, stream); break;
    default: return 2;
  }
  if (st) return st;
  const dim3 gg((unsigned)((p.tokens + 31) / 32), (unsigned)p.H);
  hipLaunchKernelGGL((bwd_pos_grad_kernel<T, false>), gg, dim3(256), 0, stream, p, d);
  hipLaunchKernelGGL((bwd_pos_grad_kernel<T, true>), gg, dim3(256), 0, stream, p, d);
  hipLaunchKernelGGL(bwd_pos_w_kernel<T>, dim3((unsigned)((2 * p.band + 1 + 63) / 64), (unsigned)p.units, (unsigned)p.H),
                     dim3(256), 0, stream, p, d);
  if (p.flags) {   // dkr / dqr exist only with a position term
    const int64_t rcells = (int64_t)p.n_rel * p.H * d;
    hipLaunchKernelGGL(bwd_pos_rel_kernel<T>, dim3((unsigned)((rcells + 255) / 256)), dim3(256), 0, stream, p, d);
  }
  return 0;
}

}  // namespace

int64_t bwd_workspace_bytes(int64_t tokens, int32_t units, int32_t H, int32_t d, int esize,
                            int32_t band) {
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t th = tokens * H;
  const int64_t wrows = 2 * (int64_t)band + 1;
  return al(th * 4) + 2 * al(th * d * 4) + 2 * al(th * 2 * 4) +
         al((int64_t)H * (2 * (int64_t)band - 1) * tokens * esize) + 2 * al((int64_t)H * units * wrows * d * 4);
}

void bwd_carve_workspace(BwdParams& p, void* ws, int d, int esize) {
  auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
  unsigned char* w = reinterpret_cast<unsigned char*>(ws);
  const int64_t th = p.tokens * p.H;
  const int64_t wrows = 2 * (int64_t)p.band + 1;
  p.dsum = reinterpret_cast<float*>(w); w += al(th * 4);
  p.dq_part = reinterpret_cast<float*>(w); w += al(th * d * 4);
  p.dk_part = reinterpret_cast<float*>(w); w += al(th * d * 4);
  p.afar = reinterpret_cast<float*>(w); w += al(th * 2 * 4);
  p.bfar = reinterpret_cast<float*>(w); w += al(th * 2 * 4);
  p.dg = w; w += al((int64_t)p.H * (2 * (int64_t)p.band - 1) * p.tokens * esize);
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
