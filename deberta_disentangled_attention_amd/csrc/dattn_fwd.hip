// Fused disentangled-attention forward for gfx950 (MI355X, CDNA4).
//
// What is computed (DisentangledFlash README "Status"; kernels-community
// discussion #31 "Motivation"): exact bidirectional DeBERTa-v2/v3 attention,
//   S_ij = tau * (q_i.k_j + q_i.kr[T(i-j)] + k_j.qr[T(j-i)]),
//   O_i  = softmax over valid keys of S_i. times V,
// streamed over key tiles with an online softmax so that no [L, L] array is
// ever stored. T is the relative-row table written by rel_bucket.
//
// Work decomposition. One workgroup of NW waves owns BM = 32*NW consecutive
// queries of one (sequence, head); wave w owns queries 32w .. 32w+31. The
// workgroup walks the keys in tiles of BN.
//
// Orientation. Every score block is produced transposed, S^T = K Q^T, by the
// 32x32 MFMA (v_mfma_f32_32x32x16_{bf16,f16} or v_mfma_f32_32x32x2_f32). In
// the MFMA result lane l holds column l%32 and rows 8(r/4) + 4(l/32) + r%4
// of register r, so each lane owns ONE query and 16 keys of a 32-key block;
// the lane pair (l, l^32) together hold all keys of that query. Row max and
// row sum are therefore per-lane scalars with a single cross-half exchange,
// and P^T is already in the register layout the P.V MFMA (O^T = V^T P^T)
// takes as its B operand - no transpose of P is needed.
//
// Position terms. For a tile, the distances i-j span a band of at most
// 32+BN-1 values per wave and BM+BN-1 per workgroup.
//  * Band path: the content-to-position products are evaluated for every
//    distance u of the wave's band, E[u][i] = q_i . kr[T(u)] (MFMA with the
//    kr rows gathered through T as the A operand), stored in LDS and read
//    back along the diagonal u = i - j. The position-to-content products
//    F[j][v] = k_j . qr[T(v)] are evaluated once per workgroup for the
//    band of v = j - i and read back the same way. Indexing the band by
//    distance (not by table row) makes every gather address affine in
//    (i, j), so the read needs no table lookup and no bank conflicts.
//  * Constant path: once |i - j| is large the table saturates and a term no
//    longer depends on the pair: C2P becomes a per-query scalar a_i, folded
//    into the softmax offset, and P2C a per-key scalar c_j, which enters as
//    the MFMA accumulator input of the Q.K product (c_j = K . qr[T]).
//    The choice is made per tile from the table values at the band ends
//    (T is monotone), so it is exact, not a heuristic.
//
// Masks. The factorised mask m_i m_j: keys with m_j = 0 (or beyond the
// sequence) get -inf scores and zero V rows; queries with m_i = 0 produce
// zero rows. Key tiles past the last valid key are never visited, and query
// tiles past it only write zeros (padded layout) or exit (packed layout).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dattn_internal.h"

namespace dattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxSeqLen = 8192;

struct TBF16 {};
struct TF16 {};
struct TF32 {};

// Per element type: storage size, how many reduction elements one lane feeds
// to one MFMA (LANE_K), the MFMA itself and the fp32 -> element rounding.
template <class T> struct Ty;

template <> struct Ty<TBF16> {
  static constexpr int ESIZE = 2;
  static constexpr int LANE_K = 8;
  typedef bf16x8_t frag;
  __device__ static __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag cvt8(f32x8_t x) {
    return __builtin_convertvector(x, bf16x8_t);
  }
};

template <> struct Ty<TF16> {
  static constexpr int ESIZE = 2;
  static constexpr int LANE_K = 8;
  typedef f16x8_t frag;
  __device__ static __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag cvt8(f32x8_t x) {
    return __builtin_convertvector(x, f16x8_t);
  }
};

template <> struct Ty<TF32> {
  static constexpr int ESIZE = 4;
  static constexpr int LANE_K = 1;
  typedef float frag;
  __device__ static __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Compile-time shape of one kernel instance.
template <class T, int D, int BN, int NW>
struct Cfg {
  static constexpr int ESIZE = Ty<T>::ESIZE;
  static constexpr int NT = 64 * NW;                 // threads
  static constexpr int BM = 32 * NW;                 // queries per workgroup
  static constexpr int NKB = BN / 32;                // 32-key blocks per tile
  static constexpr int NDB = D / 32;                 // 32-wide blocks of the head dim
  static constexpr int HALF = D / 2;                 // reduction elements per lane half
  static constexpr int NU = HALF * ESIZE / 16;       // 16-byte units per lane half-row
  static constexpr int EPU = 16 / ESIZE;             // elements per 16-byte unit
  static constexpr int NC = HALF / Ty<T>::LANE_K;    // MFMAs per d-long product
  static constexpr int NBU = BN / 32 + 1;            // C2P band blocks (per wave)
  static constexpr int NBV = NW + BN / 32;           // P2C band blocks (per workgroup)
  static constexpr int KPITCH = D + EPU;             // K tile row pitch (elements)
  static constexpr int VPITCH = BN + 4;              // V^T tile row pitch (elements)
  static constexpr int EW = 32 * NBU * 32;           // floats per wave for E
  static constexpr int FWP = 32 * NBV;               // F row pitch (floats)
  static constexpr int K_BYTES = BN * KPITCH * ESIZE;
  static constexpr int V_BYTES = D * VPITCH * ESIZE;
  static constexpr int E_BYTES = NW * EW * 4;
  static constexpr int F_BYTES = BN * FWP * 4;
  static constexpr int OFF_V = K_BYTES;
  static constexpr int OFF_E = OFF_V + V_BYTES;
  static constexpr int OFF_F = OFF_E + E_BYTES;
  static constexpr int OFF_MISC = OFF_F + F_BYTES;
  static constexpr int LDS_BYTES = OFF_MISC + 64;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU exceeded");
  static_assert(NU >= 1 && (HALF * ESIZE) % 16 == 0, "head dim too small");
  static_assert(K_BYTES % 16 == 0 && V_BYTES % 16 == 0, "alignment");
};

// ----------------------------------------------------------------------------
// small helpers
// ----------------------------------------------------------------------------

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// c-th MFMA operand inside a lane's half-row fragment held as 16-byte units
template <class T, int NU>
__device__ __forceinline__ typename Ty<T>::frag frag_at(const uint4 (&u)[NU], int c) {
  if constexpr (Ty<T>::ESIZE == 2) {
    return __builtin_bit_cast(typename Ty<T>::frag, u[c]);
  } else {
    const uint4 w = u[c >> 2];
    const uint32_t x = (c & 3) == 0 ? w.x : (c & 3) == 1 ? w.y : (c & 3) == 2 ? w.z : w.w;
    return __builtin_bit_cast(float, x);
  }
}

// acc += A . B^T over the full head dim, operands as lane half-row fragments
template <class T, int NU, int NC>
__device__ __forceinline__ f32x16_t mma_chain(const uint4 (&a)[NU], const uint4 (&b)[NU],
                                              f32x16_t acc) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
    acc = Ty<T>::mma(frag_at<T, NU>(a, c), frag_at<T, NU>(b, c), acc);
  return acc;
}

template <int NU>
__device__ __forceinline__ void load_half_row(uint4 (&u)[NU], const unsigned char* p, bool ok) {
#pragma unroll
  for (int x = 0; x < NU; ++x) u[x] = ok ? ld16(p + 16 * x) : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32); }

// ----------------------------------------------------------------------------
// the kernel
// ----------------------------------------------------------------------------

template <class T, int D, int BN, int NW, bool VARLEN>
__global__ __launch_bounds__(64 * NW) void dattn_fwd_kernel(FwdParams p) {
  typedef Cfg<T, D, BN, NW> C;
  constexpr int ES = C::ESIZE;
  constexpr int BM = C::BM;
  constexpr int NT = C::NT;
  constexpr int NU = C::NU;
  constexpr int NC = C::NC;
  constexpr float NEG_INF = -__builtin_huge_valf();

  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
  unsigned char* Ks = smem;
  unsigned char* Vt = smem + C::OFF_V;
  float* Ew_all = reinterpret_cast<float*>(smem + C::OFF_E);
  float* Fw = reinterpret_cast<float*>(smem + C::OFF_F);
  int* misc = reinterpret_cast<int*>(smem + C::OFF_MISC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;   // query column owned by this lane
  const int lh = lane >> 5;   // lane half: which 4-row groups / which k half
  float* Ew = Ew_all + wave * C::EW;

  // ---- workgroup -> (sequence, head, query tile), XCD-aware ----------------
  // Workgroups are handed to the 8 XCDs round-robin; renumber them so that
  // each XCD receives a contiguous run of logical tiles (same head and
  // sequence, hence the same K/V rows in that XCD's L2).
  const int n_work = p.n_work;
  const int hw = blockIdx.x;
  const int xcd = hw & 7;
  const int per = n_work >> 3;
  const int rem = n_work & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + (hw >> 3);

  int head, qt;
  int64_t base;        // token row of position 0 of the sequence
  int ext;             // keys/queries at positions >= ext do not exist
  int first_bad;       // first position whose mask byte is 0 (padded)
  int row_limit;       // rows < row_limit are written
  const uint8_t* mrow = nullptr;

  if (!VARLEN) {
    const int per_b = p.H * p.n_qtiles;
    const int b = logical / per_b;
    const int rest = logical - b * per_b;
    head = rest / p.n_qtiles;
    qt = rest - head * p.n_qtiles;
    base = (int64_t)b * p.L;
    row_limit = p.L;
    if (p.mask) {
      mrow = p.mask + (int64_t)b * p.L;
      if (tid == 0) { misc[0] = 0; misc[1] = p.L; }
      __syncthreads();
      int last = 0, firstz = p.L;
      for (int j = tid; j < p.L; j += NT) {
        if (mrow[j]) last = j + 1;
        else if (j < firstz) firstz = j;
      }
      if (last) atomicMax(&misc[0], last);
      if (firstz < p.L) atomicMin(&misc[1], firstz);
      __syncthreads();
      ext = misc[0];
      first_bad = misc[1];
    } else {
      ext = p.L;
      first_bad = p.L;
    }
    if (qt * BM >= ext) {
      // nothing valid in this query tile: its rows of this head are zero
      constexpr int UPR = D * ES / 16;
      const int r0 = qt * BM;
      const int nrow = min(BM, p.L - r0);
      unsigned char* o = reinterpret_cast<unsigned char*>(p.out);
      for (int x = tid; x < nrow * UPR; x += NT) {
        const int r = x / UPR, u = x - r * UPR;
        const int64_t off = ((base + r0 + r) * (int64_t)p.H * D + (int64_t)head * D) * ES + 16 * u;
        *reinterpret_cast<uint4*>(o + off) = make_uint4(0, 0, 0, 0);
      }
      return;
    }
  } else {
    head = logical / p.n_qtiles;
    const int t = logical - head * p.n_qtiles;
    // sequence b owns tile slots [floor(cu[b]/BM) + b, floor(cu[b+1]/BM) + b + 1);
    // find the last b whose first slot is <= t (256-way parallel search)
    int lo = 0, hi = p.nseq;
    while (hi - lo > 1) {
      const int span = hi - lo;
      const int step = (span + NT - 1) / NT;
      if (tid == 0) misc[2] = 0;
      __syncthreads();
      const int cand = lo + tid * step;
      if (cand < hi && tid > 0) {
        const int64_t c = min((int64_t)p.cu_seqlens[cand], p.total_tokens);
        if (c / BM + cand <= t) atomicMax(&misc[2], tid);
      }
      __syncthreads();
      const int k = misc[2];
      __syncthreads();
      lo = lo + k * step;
      hi = min(lo + step, hi);
    }
    const int b = lo;
    const int64_t c0 = max((int64_t)0, min((int64_t)p.cu_seqlens[b], p.total_tokens));
    const int64_t c1 = max(c0, min((int64_t)p.cu_seqlens[b + 1], p.total_tokens));
    qt = t - (int)(c0 / BM) - b;
    base = c0;
    ext = (int)min(c1 - c0, (int64_t)kMaxSeqLen);
    first_bad = ext;
    row_limit = ext;
    if (p.nseq <= 0 || qt < 0 || qt * BM >= ext) return;
  }

  const int i0 = qt * BM;
  const int i0w = i0 + 32 * wave;
  const bool has_c2p = (p.flags & 1u) != 0;
  const bool has_p2c = (p.flags & 2u) != 0;
  const int64_t hoff = (int64_t)head * D;  // first column of this head

  const unsigned char* Qg = reinterpret_cast<const unsigned char*>(p.q);
  const unsigned char* Kg = reinterpret_cast<const unsigned char*>(p.k);
  const unsigned char* Vg = reinterpret_cast<const unsigned char*>(p.v);
  const unsigned char* QRg = reinterpret_cast<const unsigned char*>(p.qr);
  const unsigned char* KRg = reinterpret_cast<const unsigned char*>(p.kr);

  // relative row for a signed distance (clamped reads)
  const int tbl_hi = 2 * p.rel_max_len - 2;
  auto rel_row = [&](int dist) -> int {
    int x = dist + p.rel_max_len - 1;
    x = x < 0 ? 0 : (x > tbl_hi ? tbl_hi : x);
    int r = p.rel_idx[x];
    return r < 0 ? 0 : (r >= p.n_rel ? p.n_rel - 1 : r);
  };
  auto rel_half_row = [&](const unsigned char* tab, int row) -> const unsigned char* {
    return tab + ((int64_t)row * p.ld_rel + hoff + lh * C::HALF) * ES;
  };

  // this lane's query row, half of the head dim (B operand of every product)
  uint4 qf[NU];
  {
    const int qi = i0w + li;
    const bool ok = qi < ext;
    const unsigned char* src = Qg + ((base + (ok ? qi : 0)) * p.ld_q + hoff + lh * C::HALF) * ES;
    load_half_row<NU>(qf, src, ok);
  }

  // online-softmax state of this lane's query (shared with lane ^ 32)
  float m_run = NEG_INF;
  float l_part = 0.f;
  f32x16_t o_acc[C::NDB];
#pragma unroll
  for (int x = 0; x < C::NDB; ++x) o_acc[x] = f32x16_t{};

  // constant-term caches
  int c2p_row_cached = -1;
  float a_i = 0.f;            // q_i . kr[row] for the cached row
  int p2c_row_cached = -1;
  uint4 qrc[NU];              // qr[row] half-row for the cached row
#pragma unroll
  for (int x = 0; x < NU; ++x) qrc[x] = make_uint4(0, 0, 0, 0);

  const int key_end = min(ext, first_bad);  // keys below this need no mask test

  // valid query range of the workgroup and of this wave
  const int wg_qlo = i0, wg_qhi = min(i0 + BM, ext) - 1;
  const int w_qlo = i0w, w_qhi = min(i0w + 31, ext - 1);

  for (int j0 = 0; j0 < ext; j0 += BN) {
    const bool need_mask = j0 + BN > key_end;

    // ---- stage K (row-major) and V (transposed) of the key tile ----------
    {
      constexpr int UPR = D * ES / 16;   // 16-byte units per key row
      for (int x = tid; x < BN * UPR; x += NT) {
        const int r = x / UPR, u = x - r * UPR;
        const int j = j0 + r;
        bool ok = j < ext;
        if (ok && need_mask && j >= first_bad) ok = mrow[j] != 0;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (ok) {
          kv = ld16(Kg + ((base + j) * p.ld_k + hoff) * ES + 16 * u);
          vv = ld16(Vg + ((base + j) * p.ld_v + hoff) * ES + 16 * u);
        }
        *reinterpret_cast<uint4*>(Ks + (r * C::KPITCH) * ES + 16 * u) = kv;
        const int dd0 = u * C::EPU;
        if (ES == 2) {
          uint16_t* vt = reinterpret_cast<uint16_t*>(Vt);
          const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vt[(dd0 + e) * C::VPITCH + r] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        } else {
          uint32_t* vt = reinterpret_cast<uint32_t*>(Vt);
          vt[(dd0 + 0) * C::VPITCH + r] = vv.x;
          vt[(dd0 + 1) * C::VPITCH + r] = vv.y;
          vt[(dd0 + 2) * C::VPITCH + r] = vv.z;
          vt[(dd0 + 3) * C::VPITCH + r] = vv.w;
        }
      }
    }

    // ---- choose band or constant path for each position term -------------
    const int wg_klo = j0, wg_khi = min(j0 + BN, ext) - 1;
    int p2c_mode = 0;  // 0 off, 1 constant, 2 band
    int p2c_row = 0;
    if (has_p2c) {
      const int r_lo = rel_row(wg_klo - wg_qhi), r_hi = rel_row(wg_khi - wg_qlo);
      p2c_mode = (r_lo == r_hi) ? 1 : 2;
      p2c_row = r_lo;
    }
    int c2p_mode = 0;
    int c2p_row = 0;
    if (has_c2p && w_qlo <= w_qhi) {
      const int r_lo = rel_row(w_qlo - wg_khi), r_hi = rel_row(w_qhi - wg_klo);
      c2p_mode = (r_lo == r_hi) ? 1 : 2;
      c2p_row = r_lo;
    }

    __syncthreads();  // K / V^T staged

    // ---- P2C band: F[j][v] = k_j . qr[T(vmin + v)], shared by the waves ---
    if (p2c_mode == 2) {
      const int vmin = j0 - (i0 + BM - 1);
      for (int blk = wave; blk < C::NKB * C::NBV; blk += NW) {
        const int kb = blk / C::NBV, vb = blk - kb * C::NBV;
        uint4 kf[NU], rf[NU];
#pragma unroll
        for (int x = 0; x < NU; ++x)
          kf[x] = *reinterpret_cast<const uint4*>(Ks + ((kb * 32 + li) * C::KPITCH + lh * C::HALF) * ES + 16 * x);
        const int row = rel_row(vmin + vb * 32 + li);
        load_half_row<NU>(rf, rel_half_row(QRg, row), true);
        f32x16_t acc = mma_chain<T, NU, NC>(kf, rf, f32x16_t{});
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          Fw[j * C::FWP + vb * 32 + li] = acc[r];
        }
      }
    }

    // ---- C2P band: E[u][i] = kr[T(umin + u)] . q_i, per wave --------------
    if (c2p_mode == 2) {
      const int umin = i0w - (j0 + BN - 1);
#pragma unroll
      for (int ub = 0; ub < C::NBU; ++ub) {
        uint4 rf[NU];
        const int row = rel_row(umin + ub * 32 + li);
        load_half_row<NU>(rf, rel_half_row(KRg, row), true);
        f32x16_t acc = mma_chain<T, NU, NC>(rf, qf, f32x16_t{});
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int u = ub * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          Ew[u * 32 + li] = acc[r];
        }
      }
    } else if (c2p_mode == 1 && c2p_row != c2p_row_cached) {
      // a_i = kr[row] . q_i: every A row is the same kr row
      uint4 rf[NU];
      load_half_row<NU>(rf, rel_half_row(KRg, c2p_row), true);
      f32x16_t acc = mma_chain<T, NU, NC>(rf, qf, f32x16_t{});
      a_i = acc[0];
      c2p_row_cached = c2p_row;
    }
    if (p2c_mode == 1 && p2c_row != p2c_row_cached) {
      load_half_row<NU>(qrc, rel_half_row(QRg, p2c_row), true);
      p2c_row_cached = p2c_row;
    }

    __syncthreads();  // F (and E) written

    // ---- scores -------------------------------------------------------
    f32x16_t s[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      uint4 kf[NU];
#pragma unroll
      for (int x = 0; x < NU; ++x)
        kf[x] = *reinterpret_cast<const uint4*>(Ks + ((kb * 32 + li) * C::KPITCH + lh * C::HALF) * ES + 16 * x);
      f32x16_t acc = f32x16_t{};
      if (p2c_mode == 1) acc = mma_chain<T, NU, NC>(kf, qrc, acc);  // c_j in every column
      acc = mma_chain<T, NU, NC>(kf, qf, acc);
      if (c2p_mode == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          acc[r] += Ew[(li - jj + BN - 1) * 32 + li];
        }
      }
      if (p2c_mode == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          acc[r] += Fw[jj * C::FWP + (jj - 32 * wave - li + BM - 1)];
        }
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          bool ok = j < ext;
          if (ok && j >= first_bad) ok = mrow[j] != 0;
          if (!ok) acc[r] = NEG_INF;
        }
      }
      s[kb] = acc;
    }

    // ---- online softmax (base 2, scale folded) ---------------------------
    {
      const float tl2 = p.scale_log2;
      const float off = (c2p_mode == 1) ? a_i * tl2 : 0.f;
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float mt = (mx == NEG_INF) ? NEG_INF : fmaf(mx, tl2, off);
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      const float bias = off - m_use;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], tl2, bias));
          s[kb][r] = e;
          ps += e;
        }
      l_part = fmaf(l_part, alpha, ps);
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int x = 0; x < C::NDB; ++x) o_acc[x] *= alpha;
      }
      m_run = m_new;
    }

    // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      if constexpr (ES == 2) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          f32x8_t pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = s[kb][8 * c2 + e];
          const typename Ty<T>::frag pb = Ty<T>::cvt8(pv);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const uint16_t* vrow = reinterpret_cast<const uint16_t*>(Vt) + (db * 32 + li) * C::VPITCH +
                                   kb * 32 + 16 * c2 + 4 * lh;
            const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
            const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
            const typename Ty<T>::frag va =
                __builtin_bit_cast(typename Ty<T>::frag, make_uint4(lo.x, lo.y, hi.x, hi.y));
            o_acc[db] = Ty<T>::mma(va, pb, o_acc[db]);
          }
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const float* vrow = reinterpret_cast<const float*>(Vt) + (db * 32 + li) * C::VPITCH +
                                kb * 32 + 8 * q4 + 4 * lh;
            const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(vrow);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o_acc[db] = Ty<T>::mma(vv[e], s[kb][4 * q4 + e], o_acc[db]);
          }
        }
      }
    }

    __syncthreads();  // tile buffers free for the next key tile
  }

  // ---- epilogue: normalise, zero padded rows, store ----------------------
  {
    const float l_tot = l_part + wave_xor32(l_part);
    const int qi = i0w + li;
    bool row_ok = qi < ext && l_tot > 0.f;
    if (!VARLEN && mrow && qi < ext) row_ok = row_ok && mrow[qi] != 0;
    const float inv = row_ok ? 1.f / l_tot : 0.f;
    if (qi < row_limit) {
      unsigned char* o = reinterpret_cast<unsigned char*>(p.out) +
                         ((base + qi) * (int64_t)p.H * D + hoff) * ES;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = db * 32 + 8 * g + 4 * lh;
          const float v0 = o_acc[db][4 * g + 0] * inv, v1 = o_acc[db][4 * g + 1] * inv;
          const float v2 = o_acc[db][4 * g + 2] * inv, v3 = o_acc[db][4 * g + 3] * inv;
          if constexpr (ES == 4) {
            *reinterpret_cast<f32x4_t*>(o + dd * 4) = f32x4_t{v0, v1, v2, v3};
          } else {
            f32x8_t w = f32x8_t{v0, v1, v2, v3, 0.f, 0.f, 0.f, 0.f};
            const typename Ty<T>::frag h8 = Ty<T>::cvt8(w);
            const uint4 bits = __builtin_bit_cast(uint4, h8);
            *reinterpret_cast<uint2*>(o + dd * 2) = make_uint2(bits.x, bits.y);
          }
        }
    }
  }
}

// ----------------------------------------------------------------------------
// host-side launch
// ----------------------------------------------------------------------------

template <class T, int D, int BN, int NW>
int launch_inst(FwdParams& p, bool varlen, hipStream_t stream) {
  typedef Cfg<T, D, BN, NW> C;
  int64_t n_work;
  if (!varlen) {
    p.n_qtiles = (p.L + C::BM - 1) / C::BM;
    n_work = (int64_t)p.B * p.H * p.n_qtiles;
  } else {
    p.n_qtiles = (int32_t)(p.total_tokens / C::BM + p.nseq);
    n_work = (int64_t)p.H * p.n_qtiles;
  }
  if (n_work <= 0) return 0;
  if (n_work > 0x7fffffffLL) return 2;
  p.n_work = (int32_t)n_work;
  if (varlen)
    hipLaunchKernelGGL((dattn_fwd_kernel<T, D, BN, NW, true>), dim3((unsigned)n_work), dim3(C::NT), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((dattn_fwd_kernel<T, D, BN, NW, false>), dim3((unsigned)n_work), dim3(C::NT), 0,
                       stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

template <class T>
int launch_dtype(FwdParams& p, int d, bool varlen, hipStream_t stream) {
  switch (d) {
    case 32: return launch_inst<T, 32, 64, 4>(p, varlen, stream);
    case 64: return launch_inst<T, 64, 64, 4>(p, varlen, stream);
    case 128:
      if constexpr (Ty<T>::ESIZE == 4) return launch_inst<T, 128, 32, 4>(p, varlen, stream);
      else return launch_inst<T, 128, 64, 4>(p, varlen, stream);
    default: return 2;
  }
}

int launch_fwd(FwdParams& p, int dtype, int d, bool varlen, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_dtype<TF32>(p, d, varlen, stream);
    case 1: return launch_dtype<TF16>(p, d, varlen, stream);
    case 2: return launch_dtype<TBF16>(p, d, varlen, stream);
    default: return 2;
  }
}

}  // namespace dattn
