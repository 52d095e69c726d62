// Fused disentangled-attention forward for gfx950 (MI355X, CDNA4).
//
// What is computed (DisentangledFlash README "Status"; kernels-community
// discussion #31 "Motivation"): exact bidirectional DeBERTa-v2/v3 attention,
//   S_ij = tau * (q_i.k_j + q_i.kr[T(i-j)] + k_j.qr[T(j-i)]),
//   O_i  = softmax over the valid keys of row i of S, times V,
// streamed over key tiles with an online softmax so that no [L, L] array is
// ever stored. T is the relative-row table written by rel_bucket.
//
// Work decomposition. One workgroup of NW waves owns BM = 32*NW consecutive
// queries of one (sequence, head); wave w owns queries 32w .. 32w+31. The
// workgroup walks the keys in tiles of BN, double-buffered through
// registers: the next tile's K and V rows are in flight from HBM while the
// current tile is computed from LDS.
//
// Orientation. Every score block is produced transposed, S^T = K Q^T, by the
// 32x32 MFMA (v_mfma_f32_32x32x16_{bf16,f16} or v_mfma_f32_32x32x2_f32). In
// the MFMA result lane l holds column l%32 and rows 8(r/4) + 4(l/32) + r%4
// of register r, so each lane owns ONE query and 16 keys of a 32-key block;
// the lane pair (l, l^32) together hold all keys of that query. Row max and
// row sum are per-lane scalars with a single cross-half exchange, and P^T is
// already in the register layout the P.V MFMA (O^T = V^T P^T) takes as its
// B operand - no transpose of P is needed.
//
// Position terms. The relative table is non-decreasing and saturates: beyond
// the distances sat_top / sat_bot it returns its last / first row. Those two
// thresholds are found once per workgroup, so the path of a tile is decided
// by comparing its distance range with them:
//  * constant path (every pair of the tile reads the same row): C2P is a
//    per-query scalar a_i = q_i . kr[row], folded into the softmax offset,
//    and P2C a per-key scalar c_j = k_j . qr[row], computed while the key
//    tile is staged (dot products over the lanes holding each row) and fed
//    as the accumulator input of the Q.K MFMA;
//  * band path: per 32-key half, E[u][i] = q_i . kr[T(u)] for the 63
//    distances u = i - j of the wave and F[j][v] = k_j . qr[T(v)] for the
//    distances v = j - i (the wave's 63 for 16-bit types, the workgroup's
//    BM+31 for fp32) are produced by MFMA (table rows gathered into the A/B
//    operands), stored in LDS and read back along the diagonal. Indexing the
//    bands by distance makes every gather address a per-lane base plus a
//    compile-time offset.
//
// Masks. The factorised mask m_i m_j: keys with m_j = 0 (or beyond the
// sequence) get -inf scores and zero V rows; queries with m_i = 0 produce
// zero rows. Key tiles past the last valid key are never visited, and query
// tiles past it only write zeros (padded layout) or exit (packed layout).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "dattn_device.h"
#include "dattn_internal.h"



namespace dattn {

constexpr int kMaxSeqLen = 8192;
constexpr int kShortPadded = 1024;   // padded lengths up to this order their items query tile first

// Compile-time shape of one kernel instance.
template <class T, int D, int BN, int NW>
struct Cfg {
  static constexpr int ES = Ty<T>::ESIZE;
  static constexpr int NT = 64 * NW;                 // threads
  static constexpr int BM = 32 * NW;                 // queries per workgroup
  static constexpr int NKB = BN / 32;                // 32-key blocks per tile
  static constexpr int NDB = D / 32;                 // 32-wide blocks of the head dim
  static constexpr int HALF = D / 2;                 // reduction elements per lane half
  static constexpr int NU = HALF * ES / 16;          // 16-byte units per lane half-row
  static constexpr int EPU = 16 / ES;                // elements per 16-byte unit
  static constexpr int NC = HALF / Ty<T>::LANE_K;    // MFMAs per d-long product
  static constexpr int NBV = NW + 1;                 // F blocks per 32-key half (BM+31 distances)
  static constexpr int KPITCH = D + EPU;             // K tile row pitch (elements)
  // V^T row pitch (elements). 16-bit types: BN+8, so every P.V operand is
  // one aligned 16-byte read and rows 8 apart fall 32 banks apart; fp32:
  // BN+4 (16-byte reads). With the staging order below both the reads and
  // the transposing stores are free of bank conflicts.
  static constexpr int VPITCH = ES == 2 ? BN + 8 : BN + 4;
  static constexpr int EW = 64 * 32;                 // floats of E per wave (64 distances x 32 queries)
  static constexpr int FWP = 32 * NBV;               // F row pitch (floats)
  static constexpr int UPR = D * ES / 16;            // 16-byte units per K/V row
  static constexpr int JOBS = (BN / 2) * UPR;        // staging jobs: (row pair, unit)
  static constexpr int JPT = (JOBS + NT - 1) / NT;   // jobs per thread
  // V staging: a wave moves one group per step, 16-bit types 32 row pairs x
  // 2 units, fp32 16 row pairs x 4 units
  static constexpr int VG_U = ES == 2 ? 2 : 4;       // units per group
  static constexpr int VG_P = 64 / VG_U;             // row pairs per group
  static constexpr int UG = UPR / VG_U;              // unit groups per row
  static constexpr int GROUPS = UG * (BN / 2 / VG_P); // groups per tile
  static constexpr int GPW = (GROUPS + NW - 1) / NW; // groups per wave
  static constexpr int K_BYTES = BN * KPITCH * ES;
  static constexpr int V_BYTES = (D * VPITCH * ES + 15) / 16 * 16;
  static constexpr int E_BYTES = NW * EW * 4;
  static constexpr int F_BYTES = 32 * FWP * 4;
  static constexpr int C_BYTES = BN * 4;
  static constexpr int R_BYTES = 4 * D * ES;         // qr/kr rows at both saturation ends
  static constexpr int TW = 2048;                    // table window staged in LDS (entries)
  static constexpr int TW_BYTES = TW * 4;
  static constexpr int OFF_V = K_BYTES;
  static constexpr int OFF_E = OFF_V + V_BYTES;
  static constexpr int OFF_F = OFF_E + E_BYTES;
  // far-tile ring (16-bit types): NSTAGE slots of a K tile and a V tile, both
  // dense [BN][D] rows written by direct-to-LDS loads; it reuses the region
  // of the general-tile buffers above
  static constexpr int NSTAGE = 4;
  static constexpr int KT_BYTES = BN * UPR * 16;
  static constexpr int SLOT_BYTES = 2 * KT_BYTES;
  static constexpr int RING_BYTES = ES == 2 ? NSTAGE * SLOT_BYTES : 0;
  // general tiles of 16-bit types: two slots of the ring's layout, then the
  // per-wave scratch of the band products (E: 64 distances x 32 queries, F:
  // 32 keys x 64 distances, fp32) and of the per-wave c_j
  // F rows are FPITCH floats apart: the 16x16 products store four key rows
  // 4 apart per instruction, which then fall 16 banks apart
  static constexpr int FPITCH = 68;
  static constexpr int SCR_BYTES = (64 * 32 > 32 * FPITCH ? 64 * 32 : 32 * FPITCH) * 4;
  static constexpr int OFF_SCR = 2 * SLOT_BYTES;
  static constexpr int OFF_CJW = OFF_SCR + NW * SCR_BYTES;
  static constexpr int G16_BYTES = ES == 2 ? OFF_CJW + NW * BN * 4 : 0;
  // general tiles of fp32: the register-staged layout above
  static constexpr int P1_BYTES = ES == 4 ? OFF_F + F_BYTES : 0;
  static constexpr int P_MAX = P1_BYTES > RING_BYTES ? P1_BYTES : RING_BYTES;
  static constexpr int OFF_C = P_MAX > G16_BYTES ? P_MAX : G16_BYTES;
  static constexpr int OFF_R = OFF_C + C_BYTES;
  static constexpr int OFF_TW = OFF_R + R_BYTES;
  static constexpr int OFF_MISC = OFF_TW + TW_BYTES;
  static constexpr int MISC_INTS = 8 + 4 * NW;       // scalars, then two rounds of per-wave pairs
  static constexpr int LDS_BYTES = OFF_MISC + 4 * MISC_INTS;
  // two workgroups per CU when they fit in its 160 KB of LDS
  static constexpr int WG_PER_CU = LDS_BYTES <= 80 * 1024 ? 2 : 1;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU exceeded");
  static_assert(NU >= 1 && (HALF * ES) % 16 == 0, "head dim too small");
  static_assert(K_BYTES % 16 == 0 && (OFF_E % 16) == 0 && (OFF_R % 16) == 0, "alignment");
  static_assert(BN % 32 == 0 && BN <= 64, "key tile");
  static_assert(UPR % 4 == 0 && UPR <= 32 && NT % UPR == 0, "staging groups");
  static_assert((BN / 2) % VG_P == 0, "V staging groups");
  static_assert(K_BYTES + V_BYTES + C_BYTES <= E_BYTES + F_BYTES, "second K/V buffer");
  static_assert(ES == 4 || (UPR >= 4 && UPR <= 16 && UPR % NW == 0 && BN == 64), "ring loads");
  // direct-to-LDS loads: one wave instruction moves 64 units (1 KB) of a tile
  static constexpr int DMA_PER_TILE = BN * UPR / 64;          // per K (and per V) tile
  static constexpr int DMA_PER_WAVE = DMA_PER_TILE / NW;      // per K (and per V) tile
  // XOR swizzles of the 16-byte units of ring rows. K: the 16 rows read by
  // one quarter-wave of an MFMA operand load land in distinct bank groups.
  // V: the four keys x 32 bytes of a quarter-wave transposing read do.
  __device__ static constexpr int swz_k(int r) { return (r * UPR / 16) % UPR; }
  __device__ static constexpr int swz_v(int r) {
    return UPR == 8 ? ((r >> 1) & 1) << 2 : (UPR == 16 ? (r & 3) << 2 : 0);
  }
  static_assert(V_BYTES % 16 == 0, "alignment");
};

// ----------------------------------------------------------------------------
// the kernel
// ----------------------------------------------------------------------------

enum : int { TERM_OFF = 0, TERM_CONST = 1, TERM_BAND = 2 };

// One work item: query tile qt of one (sequence, head). Every thread of the
// workgroup calls it with the same item; it may return early (uniformly).
template <class T, int D, int BN, int NW, bool VARLEN>
__device__ __forceinline__ void fwd_item(const FwdParams& p, int item, unsigned char* smem) {
  typedef Cfg<T, D, BN, NW> C;
  constexpr int ES = C::ES;
  constexpr int BM = C::BM;
  constexpr int NT = C::NT;
  constexpr int NU = C::NU;
  constexpr int NC = C::NC;
  constexpr float NEG_INF = -__builtin_huge_valf();

  unsigned char* Ks = smem;
  unsigned char* Vt = smem + C::OFF_V;
  float* Ew = reinterpret_cast<float*>(smem + C::OFF_E);
  float* Fw = reinterpret_cast<float*>(smem + C::OFF_F);
  float* cbuf = reinterpret_cast<float*>(smem + C::OFF_C);
  unsigned char* Rrows = smem + C::OFF_R;   // qr_top, qr_bot, kr_top, kr_bot
  int* misc = reinterpret_cast<int*>(smem + C::OFF_MISC);
  uint32_t* Tw = reinterpret_cast<uint32_t*>(smem + C::OFF_TW);   // row offsets of a window of distances

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;   // query column owned by this lane
  const int lh = lane >> 5;   // lane half: which 4-row groups / which k half
  float* Eww = Ew + wave * C::EW;

  // ---- item -> (sequence, head, query tile), XCD-aware ----------------------
  // Items are handed to the 8 XCDs round-robin; renumber them so that each
  // XCD receives a contiguous run of logical tiles (same head and sequence,
  // hence the same K/V rows in that XCD's L2). With qt_major (short padded
  // batches with a mask) the query tile varies slowest instead, so the
  // tiles that hold valid queries of right-padded rows are dispatched first
  // and the zero-only ones last; K/V of short rows are small enough that no
  // XCD grouping is needed.
  const int n_work = p.n_work;
  const int hw = item;
  const int xcd = hw & 7;
  const int per = n_work >> 3;
  const int rem = n_work & 7;
  const int logical = p.qt_major ? hw : xcd * per + (xcd < rem ? xcd : rem) + (hw >> 3);

  int head, qt;
  int64_t base;        // token row of position 0 of the sequence
  int ext;             // keys/queries at positions >= ext do not exist
  int first_bad;       // first position whose mask byte is 0 (padded)
  int row_limit;       // rows < row_limit are written
  const uint8_t* mrow = nullptr;

  if (!VARLEN) {
    int b;
    if (p.qt_major) {
      const int per_qt = p.B * p.H;
      qt = logical / per_qt;
      const int rest = logical - qt * per_qt;
      b = rest / p.H;
      head = rest - b * p.H;
    } else {
      const int per_b = p.H * p.n_qtiles;
      b = logical / per_b;
      const int rest = logical - b * per_b;
      head = rest / p.n_qtiles;
      qt = rest - head * p.n_qtiles;
    }
    base = (int64_t)b * p.L;
    row_limit = p.L;
    if (p.mask) {
      // Every wave scans the whole mask row and reduces it itself (no
      // barrier): ext = one past the last valid position, first_bad = the
      // first padded one. A query tile with no valid query at or after its
      // first row (most tiles of a heavily padded batch) then has
      // qt * BM >= ext and leaves below.
      mrow = p.mask + (int64_t)b * p.L;
      int last = 0, firstz = p.L;
      // loads in batches of 8 per lane, so that a batch costs one round trip
      constexpr int MB = 8;
      if ((p.L & 3) == 0 && (reinterpret_cast<uintptr_t>(mrow) & 3) == 0) {
        const uint32_t* mw = reinterpret_cast<const uint32_t*>(mrow);
        const int nw = p.L >> 2;
        for (int w0 = 0; w0 < nw; w0 += 64 * MB) {
          uint32_t m4[MB];
#pragma unroll
          for (int k = 0; k < MB; ++k) {
            const int w = w0 + lane + 64 * k;
            m4[k] = mw[min(w, nw - 1)];   // unconditional: the loads issue together
          }
#pragma unroll
          for (int k = 0; k < MB; ++k) {
            const int w = w0 + lane + 64 * k;
            if (w < nw) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int j = 4 * w + e;
                if ((m4[k] >> (8 * e)) & 0xffu) last = j + 1;
                else firstz = min(firstz, j);
              }
            }
          }
        }
      } else {
        for (int j0 = 0; j0 < p.L; j0 += 64 * MB) {
          uint8_t m1[MB];
#pragma unroll
          for (int k = 0; k < MB; ++k) {
            const int j = j0 + lane + 64 * k;
            m1[k] = mrow[min(j, p.L - 1)];
          }
#pragma unroll
          for (int k = 0; k < MB; ++k) {
            const int j = j0 + lane + 64 * k;
            if (j < p.L) {
              if (m1[k]) last = j + 1;
              else firstz = min(firstz, j);
            }
          }
        }
      }
      ext = wave_max_i(last);
      first_bad = wave_min_i(firstz);
    } else {
      ext = p.L;
      first_bad = p.L;
    }
    if (qt * BM >= ext) {
      // nothing valid in this query tile: its rows of this head are zero
      const int r0 = qt * BM;
      const int nrow = min(BM, p.L - r0);
      unsigned char* o = reinterpret_cast<unsigned char*>(p.out);
      for (int x = tid; x < nrow * C::UPR; x += NT) {
        const int r = x / C::UPR, u = x - r * C::UPR;
        const int64_t off = ((base + r0 + r) * (int64_t)p.H * D + (int64_t)head * D) * ES + 16 * u;
        *reinterpret_cast<uint4*>(o + off) = make_uint4(0, 0, 0, 0);
      }
      if (p.lse)
        for (int r = tid; r < nrow; r += NT) p.lse[(base + r0 + r) * p.H + head] = NEG_INF;
      return;
    }
  } else {
    head = logical / p.n_qtiles;
    const int t = logical - head * p.n_qtiles;
    // sequence b owns tile slots [floor(cu[b]/BM) + b, floor(cu[b+1]/BM) + b + 1);
    // find the last b whose first slot is <= t, i.e. the first b whose first
    // slot is > t, minus one
    const int nb = p.nseq;
    const int64_t tot = p.total_tokens;
    const int32_t* cu = p.cu_seqlens;
    const int first_after = block_first_true<NT>(
        nb, [&](int b) { return min((int64_t)cu[b], tot) / BM + b > t; }, &misc[2], tid);
    const int b = max(first_after - 1, 0);
    const int64_t c0 = max((int64_t)0, min((int64_t)cu[b], tot));
    const int64_t c1 = max(c0, min((int64_t)cu[b + 1], tot));
    qt = t - (int)(c0 / BM) - b;
    base = c0;
    ext = (int)min(c1 - c0, (int64_t)kMaxSeqLen);
    first_bad = ext;
    row_limit = ext;
    if (qt < 0 || qt * BM >= ext) return;
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

  // ---- relative table: saturation thresholds and rows ---------------------
  const int R = p.rel_max_len;
  const int tbl_n = 2 * R - 1;
  auto clamp_row = [&](int r) { return r < 0 ? 0 : (r >= p.n_rel ? p.n_rel - 1 : r); };
  // byte offset of a (clamped) relative row; rows times the row stride fit in
  // 31 bits (checked by the host)
  const uint32_t ld_rel_b = (uint32_t)(p.ld_rel * ES);
  auto row_off = [&](int r) { return (uint32_t)clamp_row(r) * ld_rel_b; };
  int sat_top = 1 << 30, sat_bot = -(1 << 30);
  int row_hi = 0, row_lo = 0;
  int tw0 = 0, tw_n = 1;   // staged window: distances tw0 .. tw0 + tw_n - 1
  bool tw_ok = false;
  // Byte offset of the qr / kr row of a signed distance. The table is
  // staged in LDS as offsets for a window of distances that contains
  // sat_bot .. sat_top (its end entries stand for everything beyond), or
  // read from global memory when that window is too long; the two cases
  // are separate instantiations of the general-tile loops, so the common
  // one never waits on a global load.
  auto rel_off = [&](int dist, auto twok) -> uint32_t {
    if constexpr (decltype(twok)::value) {
      return Tw[min(max(dist - tw0, 0), tw_n - 1)];
    } else {
      int r;
      if (dist <= sat_bot) r = row_lo;
      else if (dist >= sat_top) r = row_hi;
      else {
        int x = dist + R - 1;
        x = x < 0 ? 0 : (x > tbl_n - 1 ? tbl_n - 1 : x);
        r = p.rel_idx[x];
      }
      return row_off(r);
    }
  };
  // this lane's query row, half of the head dim (B operand of every
  // product); issued first so that its latency overlaps the table's
  uint4 qf[NU];
  {
    const int qi = i0w + li;
    if (qi < ext) {
      load_half_row<NU>(qf, Qg + ((base + qi) * p.ld_q + hoff + lh * C::HALF) * ES);
    } else {
#pragma unroll
      for (int x = 0; x < NU; ++x) qf[x] = make_uint4(0, 0, 0, 0);
    }
  }

  if (has_c2p || has_p2c) {
    // The table is non-decreasing, so both thresholds (the first index that
    // holds its last value, the first that leaves its first value) are
    // bracketed by NT samples spaced `step` apart (the last one at n-1) and
    // then settled exactly by the entries inside the two brackets. The
    // window staged in LDS is the union of the two brackets and everything
    // between them: its end entries are saturated, so clamping an index
    // into it reproduces the table beyond the thresholds. A table that fits
    // the window buffer is read whole together with the samples (one round
    // of loads); a longer one is read in a second round, the window only.
    // Cross-wave results go through per-wave LDS slots, one barrier each.
    const int32_t* tb = p.rel_idx;
    const int step = tbl_n > 1 ? (tbl_n - 2) / (NT - 1) + 1 : 1;
    constexpr int TPT = C::TW / NT;   // entries per thread of a whole table
    const bool whole = tbl_n <= C::TW;
    row_hi = tb[tbl_n - 1];
    row_lo = tb[0];
    const int vs = tb[min(tid * step, tbl_n - 1)];
    int ent[TPT];
    const int nk = (tbl_n + NT - 1) / NT;   // chunks of NT entries a whole table has
    if (whole) {
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int x = tid + k * NT;
        ent[k] = k < nk ? tb[min(x, tbl_n - 1)] : 0;
      }
    }
    // minimum over the workgroup of a wave-reduced pair, through slots at o
    auto block_min2 = [&](int a, int b, int o) -> int2 {
      if (lane == 0) { misc[o + 2 * wave] = a; misc[o + 2 * wave + 1] = b; }
      __syncthreads();
      int2 r = make_int2(misc[o], misc[o + 1]);
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        r.x = min(r.x, misc[o + 2 * w]);
        r.y = min(r.y, misc[o + 2 * w + 1]);
      }
      return make_int2(__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y));
    };
    // first sample holding the last value (exists: the last sample is n-1)
    // and first sample leaving the first value (NT: none, a flat table)
    const int2 tt = block_min2(wave_min_i(vs == row_hi ? tid : NT), wave_min_i(vs != row_lo ? tid : NT), 8);
    const int t_top = tt.x, t_bot = tt.y;
    // brackets: first_top in (lo_top, hi_top], first_above_bot in (lo_bot, hi_bot]
    const int hi_top = min(t_top * step, tbl_n - 1);
    const int lo_top = t_top > 0 ? min((t_top - 1) * step, tbl_n - 1) : -1;
    const bool flat = t_bot >= NT;                  // every entry equals the first
    const int hi_bot = flat ? tbl_n : min(t_bot * step, tbl_n - 1);
    const int lo_bot = flat ? tbl_n - 1 : (t_bot > 0 ? min((t_bot - 1) * step, tbl_n - 1) : -1);
    // window: table entries lo_bot .. hi_top (clamped into the table); it
    // contains both brackets
    const int w0 = max(lo_bot, 0), w1 = max(hi_top, w0);
    tw0 = w0 - (R - 1);
    tw_n = w1 - w0 + 1;
    tw_ok = !flat && tw_n <= C::TW;
    int ftop = tbl_n, fbot = tbl_n;
    auto settle = [&](int x, int v) {
      if (x > lo_top && x < hi_top && v == row_hi) ftop = min(ftop, x);
      if (!flat && x > lo_bot && x < hi_bot && v != row_lo) fbot = min(fbot, x);
    };
    if (whole) {
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int x = tid + k * NT;
        if (k < nk && x < tbl_n) {
          settle(x, ent[k]);
          if (tw_ok && x >= w0 && x <= w1) Tw[x - w0] = row_off(ent[k]);
        }
      }
    } else if (tw_ok) {
      for (int x = tid; x < tw_n; x += NT) {
        const int v = tb[w0 + x];
        Tw[x] = row_off(v);
        settle(w0 + x, v);
      }
    } else {
      // window too long to stage: the two brackets only (at most `step`
      // entries each)
      for (int k = tid; k < step; k += NT) {
        const int xt = lo_top + 1 + k, xb = lo_bot + 1 + k;
        if (xt < hi_top) settle(xt, tb[xt]);
        if (!flat && xb < hi_bot) settle(xb, tb[xb]);
      }
    }
    // stage the two saturation rows of qr and kr (this head) in LDS
    constexpr int RU = D * ES / 16;
    for (int x = tid; x < 4 * RU; x += NT) {
      const int which = x / RU, u = x - which * RU;
      const unsigned char* tab = (which < 2) ? QRg : KRg;
      const int row = clamp_row((which & 1) ? row_lo : row_hi);
      *reinterpret_cast<uint4*>(Rrows + which * D * ES + 16 * u) =
          ld16(tab + ((int64_t)row * p.ld_rel + hoff) * ES + 16 * u);
    }
    // (this barrier also publishes the window and the saturation rows)
    const int2 ff = block_min2(wave_min_i(ftop), wave_min_i(fbot), 8 + 2 * NW);
    const int first_top = min(ff.x, hi_top);
    const int first_above_bot = flat ? tbl_n : min(ff.y, hi_bot);
    sat_top = first_top - (R - 1);
    sat_bot = first_above_bot - 1 - (R - 1);
  }

  // a_i at both saturation ends: kr[row] . q_i with every A row equal
  float a_top = 0.f, a_bot = 0.f;
  if (has_c2p) {
    uint4 rf[NU];
    lds_half_row<NU>(rf, Rrows + 2 * D * ES + lh * C::HALF * ES);
    a_top = mma_chain<T, NU, NC>(rf, qf, f32x16_t{})[0];
    lds_half_row<NU>(rf, Rrows + 3 * D * ES + lh * C::HALF * ES);
    a_bot = mma_chain<T, NU, NC>(rf, qf, f32x16_t{})[0];
  }

  // online-softmax state of this lane's query (shared with lane ^ 32)
  float m_run = NEG_INF;
  float l_part = 0.f;
  f32x16_t o_acc[C::NDB];
#pragma unroll
  for (int x = 0; x < C::NDB; ++x) o_acc[x] = f32x16_t{};

  const int key_end = min(ext, first_bad);  // keys below this need no mask test
  const int wg_qlo = i0, wg_qhi = min(i0 + BM, ext) - 1;
  const int w_qlo = i0w, w_qhi = min(i0w + 31, ext - 1);

  // ---- K/V staging through registers --------------------------------------
  // K: job x = tid + s*NT covers row pair x / UPR, 16-byte unit x % UPR, so
  // the UPR lanes of a pair hold whole rows (coalesced loads, and the P2C
  // constant c_j of a row is a sum over those lanes). V: a wave's step moves
  // one group, row pairs 16*pg + lane%16 and unit 4*ug + lane/16, whose
  // transposing dword stores (one dword = the same element of both rows of
  // a pair) are free of bank conflicts.
  uint4 pk[C::JPT][2], pv[C::GPW][2];
  auto vjob_of = [&](int s, int& pr, int& u) -> bool {
    const int g = wave + NW * s;
    const int ug = g % C::UG, pg = g / C::UG;
    u = C::VG_U * ug + lane / C::VG_P;
    pr = C::VG_P * pg + lane % C::VG_P;
    return g < C::GROUPS;
  };
  // Rows of keys past the sequence are never read. Rows of masked keys are
  // read and zeroed when staged; the tile's mask bytes (key j0 + lane) are
  // fetched with it, one per lane, and turned into a 64-bit valid-key word.
  int mbyte = 1;
  auto fetch = [&](int j0) {
#pragma unroll
    for (int s = 0; s < C::JPT; ++s) {
      const int x = tid + s * NT;
      const int pr = x / C::UPR, u = x % C::UPR;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = j0 + 2 * pr + h;
        pk[s][h] = (x < C::JOBS && j < ext) ? ld16(Kg + ((base + j) * p.ld_k + hoff) * ES + 16 * u)
                                            : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < C::GPW; ++s) {
      int pr, u;
      const bool live = vjob_of(s, pr, u);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = j0 + 2 * pr + h;
        pv[s][h] = (live && j < ext) ? ld16(Vg + ((base + j) * p.ld_v + hoff) * ES + 16 * u)
                                     : make_uint4(0, 0, 0, 0);
      }
    }
    if (!VARLEN && mrow && j0 + BN > key_end) {
      const int j = j0 + lane;
      mbyte = (j < ext && j >= first_bad) ? (int)mrow[j] : 1;
    }
  };
  // bit k: key j0 + k exists and is not masked (tile last fetched by fetch)
  auto tile_valid = [&](int j0) -> uint64_t {
    return (uint64_t)__ballot(j0 + lane < ext && mbyte != 0);
  };
  // fetch for tiles known to hold only valid keys: a uniform tile base plus
  // per-thread byte offsets that do not change from tile to tile
  uint32_t koff[C::JPT][2], voff[C::GPW][2];
#pragma unroll
  for (int s = 0; s < C::JPT; ++s) {
    const int x = min(tid + s * NT, C::JOBS - 1);
    const int pr = x / C::UPR, u = x % C::UPR;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      koff[s][h] = (uint32_t)(((2 * pr + h) * p.ld_k + hoff) * ES + 16 * u);
  }
#pragma unroll
  for (int s = 0; s < C::GPW; ++s) {
    int pr, u;
    vjob_of(s, pr, u);
    pr = min(pr, BN / 2 - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      voff[s][h] = (uint32_t)(((2 * pr + h) * p.ld_v + hoff) * ES + 16 * u);
  }
  auto fetch_valid = [&](int j0) {   // requires j0 + BN <= key_end
    const unsigned char* kt = Kg + (base + j0) * p.ld_k * ES;
    const unsigned char* vt = Vg + (base + j0) * p.ld_v * ES;
#pragma unroll
    for (int s = 0; s < C::JPT; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) pk[s][h] = ld16(kt + koff[s][h]);
#pragma unroll
    for (int s = 0; s < C::GPW; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) pv[s][h] = ld16(vt + voff[s][h]);
  };
  // stage into the given K / V^T / c_j buffers; cj_which >= 0: also write
  // c_j = k_j . qr[row] (row: 0 top, 1 bottom) of the staged keys
  // kvalid: valid keys of the tile (all ones: nothing to zero)
  auto stage = [&](unsigned char* Ks, unsigned char* Vt, float* cbuf, int cj_which, uint64_t kvalid) {
    const bool zero_rows = kvalid != ~0ull;   // uniform
    auto keep = [&](int k) { return ((kvalid >> k) & 1ull) != 0; };
    if (zero_rows) {
#pragma unroll
      for (int s = 0; s < C::JPT; ++s) {
        const int pr = (tid + s * NT) / C::UPR;
        if (!keep(2 * pr)) pk[s][0] = make_uint4(0, 0, 0, 0);
        if (!keep(2 * pr + 1)) pk[s][1] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < C::GPW; ++s) {
        int pr, u;
        vjob_of(s, pr, u);
        if (!keep(2 * pr)) pv[s][0] = make_uint4(0, 0, 0, 0);
        if (!keep(2 * pr + 1)) pv[s][1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < C::JPT; ++s) {
      const int x = tid + s * NT;
      const int pr = x / C::UPR, u = x % C::UPR;
      if (x < C::JOBS) {
        *reinterpret_cast<uint4*>(Ks + ((2 * pr) * C::KPITCH) * ES + 16 * u) = pk[s][0];
        *reinterpret_cast<uint4*>(Ks + ((2 * pr + 1) * C::KPITCH) * ES + 16 * u) = pk[s][1];
      }
      if (cj_which >= 0) {   // uniform; every lane joins the group sums
        const uint4 r = *reinterpret_cast<const uint4*>(Rrows + cj_which * D * ES + 16 * u);
        const float c0 = group_sum<C::UPR>(dot16<T>(pk[s][0], r));
        const float c1 = group_sum<C::UPR>(dot16<T>(pk[s][1], r));
        if (u == 0 && x < C::JOBS) *reinterpret_cast<float2*>(cbuf + 2 * pr) = make_float2(c0, c1);
      }
    }
#pragma unroll
    for (int s = 0; s < C::GPW; ++s) {
      int pr, u;
      if (vjob_of(s, pr, u)) {
        const uint32_t a4[4] = {pv[s][0].x, pv[s][0].y, pv[s][0].z, pv[s][0].w};
        const uint32_t b4[4] = {pv[s][1].x, pv[s][1].y, pv[s][1].z, pv[s][1].w};
        if constexpr (ES == 2) {
          // element e of both rows -> one dword of V^T row (8u + e), at the
          // pair's position in the operand order (see v_pos)
          uint32_t* vt = reinterpret_cast<uint32_t*>(Vt);
          const int pp = v_pos(2 * pr) >> 1;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // bytes of the 16-bit element e of row 2pr (low) and of row 2pr+1 (high)
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            vt[(((8 * u + e) * C::VPITCH) >> 1) + pp] =
                __builtin_amdgcn_perm(b4[e >> 1], a4[e >> 1], sel);
          }
        } else {
          uint2* vt = reinterpret_cast<uint2*>(Vt);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            vt[((4 * u + e) * C::VPITCH + 2 * pr) >> 1] = make_uint2(a4[e], b4[e]);
        }
      }
    }
  };

  // per-lane V^T operand bases: row dd = li of each 32-row block; 16-bit types
  // read columns 8*lh.. of each 16-key group, fp32 keys 4*lh..
  constexpr int V_LANE = ES == 2 ? 8 : 4;
  const unsigned char* v_base0 = Vt + (li * C::VPITCH + V_LANE * lh) * ES;
  // per-lane gather bases (see the band writes below)
  const float* e_base = Eww + (li - 4 * lh + 4) * 32 + li;
  const float* f_base = Fw + 4 * lh * (C::FWP + 1) + (BM - 1 - 32 * wave - li);
  // second K/V buffer of the far phase, in the band region (unused there)
  unsigned char* Ks1 = smem + C::OFF_E;
  unsigned char* Vt1 = Ks1 + C::K_BYTES;
  float* cbuf1 = reinterpret_cast<float*>(Vt1 + C::V_BYTES);
  const unsigned char* v_base1 = Vt1 + (li * C::VPITCH + V_LANE * lh) * ES;

  // V^T operands from a staged (transposed) V tile
  auto vop_staged = [&](const unsigned char* v_base) {
    return [=](int kb, int c, int db) {
      if constexpr (ES == 2)
        return __builtin_bit_cast(typename Ty<T>::frag,
                                  ld16(v_base + (db * 32 * C::VPITCH + kb * 32 + 16 * c) * ES));
      else
        return *reinterpret_cast<const f32x4_t*>(v_base + (db * 32 * C::VPITCH + kb * 32 + 8 * c) * ES);
    };
  };

  // accumulator input of the Q.K product: c_j of the constant P2C path
  auto c_init = [&](const float* cb_base, int kb) -> f32x16_t {
    const f32x4_t* cb = reinterpret_cast<const f32x4_t*>(cb_base + kb * 32 + 4 * lh);
    const f32x4_t c0 = cb[0], c1 = cb[2], c2 = cb[4], c3 = cb[6];
    const f32x8_t c01 = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
    const f32x8_t c23 = __builtin_shufflevector(c2, c3, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_shufflevector(c01, c23, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  };

  // scores of a tile with no mask test and no band term: straight-line body
  auto far_scores = [&](f32x16_t (&s)[C::NKB], const unsigned char* kbuf, const float* cb,
                        auto p2c_const) {
    constexpr bool PC = decltype(p2c_const)::value;
    if constexpr (ES == 4) {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        f32x16_t acc = f32x16_t{};
        if constexpr (PC) acc = c_init(cb, kb);
        s[kb] = mma_chain_lds<T, NU, NC>(kbuf + ((kb * 32 + li) * C::KPITCH + lh * C::HALF) * ES, qf,
                                         acc);
      }
    } else {
      uint4 kf[C::NKB][NU];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
        lds_half_row<NU>(kf[kb], kbuf + ((kb * 32 + li) * C::KPITCH + lh * C::HALF) * ES);
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        f32x16_t acc = f32x16_t{};
        if constexpr (PC) acc = c_init(cb, kb);
        s[kb] = mma_chain<T, NU, NC>(kf[kb], qf, acc);
      }
    }
  };

  // Online softmax of a tile's scores (softmax_p) and O^T += V^T P^T (pv_acc).
  // softmax_p writes P to pfrag (16-bit types) or over s (fp32).
  // mid(): MFMA work issued in the same block as the exponentials (in the
  // pipelined far loop: the previous tile's P.V and a later tile's Q.K).
  // rescore(s): forms the tile's scores again (far loop), or nullptr.
  // vop(kb, c, db): V^T operand of the P.V MFMA for key block kb, 16-key
  // group c (16-bit types) or 8-key group c (fp32), head-dim block db.
  typedef typename Ty<T>::frag PFrag[ES == 2 ? C::NKB : 1][2];
  auto softmax_p = [&](f32x16_t (&s)[C::NKB], float a_off, PFrag& pfrag, auto mid, auto rescore) {
    // ---- online softmax (base 2, scale folded) ---------------------------
    // The exponent offset m_run follows the row maximum loosely: it is
    // raised (and the accumulators rescaled by alpha) only when a tile's
    // maximum exceeds it by more than 8. O and l share the offset, so O / l
    // does not depend on that choice. For 16-bit types the tile maximum is
    // not formed on the hot path: the exponentials are taken against the
    // current offset and their row-half sum, which is at most 32 * 2^8 when
    // no raise is due, detects a due raise (or an overflow); that rare case
    // and the first tile (no offset yet) take the cold path, which forms the
    // maximum and redoes the exponentials. The two lanes of a query always
    // move m_run together. For 16-bit types the row sum is taken from the
    // rounded P the P.V product uses (dot2 against (1, 1)).
    {
      const float tl2 = p.scale_log2;
      const float off = a_off * tl2;
      // raise m_run where this tile's maximum exceeds it by more than 8
      auto raise_to_max = [&] {
        float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            mx4[0] = fmaxf(mx4[0], s[kb][r]);
            mx4[1] = fmaxf(mx4[1], s[kb][r + 1]);
            mx4[2] = fmaxf(mx4[2], s[kb][r + 2]);
            mx4[3] = fmaxf(mx4[3], s[kb][r + 3]);
          }
        const float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
        const float mxf = fmaxf(mx, wave_xor32(mx));
        const float mt = (mxf == NEG_INF) ? NEG_INF : fmaf(mxf, tl2, off);
        const bool raise = mt > m_run + 8.f;
        const float m_new = raise ? mt : m_run;
        // m_run == -inf: nothing accumulated yet, alpha = exp2(-inf) = 0
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_part *= alpha;
#pragma unroll
        for (int x = 0; x < C::NDB; ++x) o_acc[x] *= alpha;
        m_run = m_new;
      };
      // P = exp2(s * tl2 + bias) (rounded to the element type for 16-bit
      // types); returns this lane's sum of it
      auto exps = [&]() -> float {
        const float bias = off - (m_run == NEG_INF ? 0.f : m_run);
        float ps4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            f32x8_t e8;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              e8[e] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * c2 + e], tl2, bias));
            if constexpr (ES == 2) {
              pfrag[kb][c2] = Ty<T>::cvt8(e8);
              const uint4 w = __builtin_bit_cast(uint4, pfrag[kb][c2]);
              ps4[0] = Ty<T>::sum2(w.x, ps4[0]);
              ps4[1] = Ty<T>::sum2(w.y, ps4[1]);
              ps4[2] = Ty<T>::sum2(w.z, ps4[2]);
              ps4[3] = Ty<T>::sum2(w.w, ps4[3]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                s[kb][8 * c2 + e] = e8[e];
                ps4[e & 3] += e8[e];
              }
            }
          }
        return (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      };
      constexpr bool LAZY = ES == 2 && !std::is_same<decltype(rescore), std::nullptr_t>::value;
      if constexpr (LAZY) {
        // rescore(s) forms this tile's scores again, so the scores need not
        // stay live past the exponentials; mid()'s MFMAs, the exponentials
        // and the test share one block (a lane with no offset yet always
        // takes the cold path, after mid()'s P.V has accumulated)
        mid();
        float ps = exps();
        if (__builtin_expect(__any(!(ps <= 32.f * 256.f) || m_run == NEG_INF), 0)) {
          rescore(s);
          raise_to_max();
          ps = exps();
        }
        l_part += ps;
      } else {
        // the tile maximum first: a raise is rare, so only a lane's own half
        // of the row is tested on the hot path
        float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            mx4[0] = fmaxf(mx4[0], s[kb][r]);
            mx4[1] = fmaxf(mx4[1], s[kb][r + 1]);
            mx4[2] = fmaxf(mx4[2], s[kb][r + 2]);
            mx4[3] = fmaxf(mx4[3], s[kb][r + 3]);
          }
        const float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
        const float mt_half = (mx == NEG_INF) ? NEG_INF : fmaf(mx, tl2, off);
        if (__builtin_expect(__any(mt_half > m_run + 8.f), 0)) raise_to_max();
        mid();
        l_part += exps();
      }
    }
  };

  // O^T += V^T P^T; P in pfrag (16-bit types) or in s (fp32)
  auto pv_acc = [&](const PFrag& pfrag, f32x16_t (&s)[C::NKB], auto vop) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      if constexpr (ES == 2) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const typename Ty<T>::frag pb = pfrag[kb][c2];
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            o_acc[db] = Ty<T>::mma(vop(kb, c2, db), pb, o_acc[db]);
          }
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const f32x4_t vv = vop(kb, q4, db);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o_acc[db] = Ty<T>::mma(vv[e], s[kb][4 * q4 + e], o_acc[db]);
          }
        }
      }
    }
  };
  auto softmax_pv_mid = [&](f32x16_t (&s)[C::NKB], float a_off, auto vop, auto mid, auto rescore) {
    PFrag pfrag;
    softmax_p(s, a_off, pfrag, mid, rescore);
    pv_acc(pfrag, s, vop);
  };
  auto softmax_pv = [&](f32x16_t (&s)[C::NKB], float a_off, auto vop) {
    softmax_pv_mid(s, a_off, vop, [] {}, nullptr);
  };

  // Online softmax and P.V of one 32-key half of a tile (16-bit types, 16
  // scores per lane): the offset rule of softmax_p (raise only past a margin
  // of 8); P rounded to the element type, its row sum taken from the rounded
  // values.
  auto softmax_pv_half = [&](f32x16_t& sv, int kb, float a_off, auto vop) {
    if constexpr (ES == 2) {
      const float tl2 = p.scale_log2;
      const float off = a_off * tl2;
      typename Ty<T>::frag pf[2];
      // P = exp2(s tl2 + off - m_run), rounded; returns this lane's sum of it
      auto exps = [&]() -> float {
        const float bias = off - (m_run == NEG_INF ? 0.f : m_run);
        float ps4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          f32x8_t e8;
#pragma unroll
          for (int e = 0; e < 8; ++e) e8[e] = __builtin_amdgcn_exp2f(fmaf(sv[8 * c2 + e], tl2, bias));
          pf[c2] = Ty<T>::cvt8(e8);
          const uint4 w = __builtin_bit_cast(uint4, pf[c2]);
          ps4[0] = Ty<T>::sum2(w.x, ps4[0]);
          ps4[1] = Ty<T>::sum2(w.y, ps4[1]);
          ps4[2] = Ty<T>::sum2(w.z, ps4[2]);
          ps4[3] = Ty<T>::sum2(w.w, ps4[3]);
        }
        return (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      };
      // Lazy offset: the exponentials are taken against the current m_run;
      // their sum, at most 16 * 2^8 when no value exceeds m_run by more
      // than 8, detects a due raise (or an overflow). That rare case, and
      // a lane with no offset yet, take the cold path: the half's maximum
      // (both lanes of the query), the raise with its rescale, and the
      // exponentials again.
      float ps = exps();
      if (__builtin_expect(__any(!(ps <= 16.f * 256.f) || m_run == NEG_INF), 0)) {
        float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          mx4[0] = fmaxf(mx4[0], sv[r]);
          mx4[1] = fmaxf(mx4[1], sv[r + 1]);
          mx4[2] = fmaxf(mx4[2], sv[r + 2]);
          mx4[3] = fmaxf(mx4[3], sv[r + 3]);
        }
        const float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
        const float mxf = fmaxf(mx, wave_xor32(mx));
        const float mt = (mxf == NEG_INF) ? NEG_INF : fmaf(mxf, tl2, off);
        const bool raise = mt > m_run + 8.f;
        const float m_new = raise ? mt : m_run;
        // m_run == -inf: nothing accumulated yet, alpha = exp2(-inf) = 0
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_part *= alpha;
#pragma unroll
        for (int x = 0; x < C::NDB; ++x) o_acc[x] *= alpha;
        m_run = m_new;
        ps = exps();
      }
      l_part += ps;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) o_acc[db] = Ty<T>::mma(vop(kb, c2, db), pf[c2], o_acc[db]);
    }
  };

  // ---- tile classes -------------------------------------------------------
  // Tiles before tm need no mask test. A tile is "far" when every pair of it
  // lies beyond the saturation distances of each enabled term, on the side
  // where keys precede the queries (tiles < FL) or follow them (FR <= t < tm).
  // Other tiles ("general": [FL, FR) and [tm, ntiles)) run first, through
  // the single-buffered path with band products; far tiles then reuse the
  // band region of LDS as a second K/V buffer, one barrier per tile.
  const int ntiles = (ext + BN - 1) / BN;
  const int tm = key_end >= BN ? (key_end - BN) / BN + 1 : 0;
  constexpr int BIG = 1 << 29;
  const int lim_l = wg_qlo - BN + 1 + min(has_p2c ? sat_bot : BIG, has_c2p ? -sat_top : BIG);
  const int lim_r = wg_qhi + max(has_p2c ? sat_top : -BIG, has_c2p ? -sat_bot : -BIG);
  const int FL = lim_l >= 0 ? min(lim_l / BN + 1, tm) : 0;
  const int FR = min(max(lim_r > 0 ? (lim_r + BN - 1) / BN : 0, FL), tm);
  auto next_general = [&](int t) {
    int n = t + 1;
    if (n >= FR && n < tm) n = tm;
    return n < ntiles ? n : -1;
  };
  auto next_far = [&](int t) {
    int n = t + 1;
    if (n >= FL && n < FR) n = FR;
    return n < tm ? n : -1;
  };
  const int first_general = FL < FR ? FL : (tm < ntiles ? tm : -1);
  const int first_far = FL > 0 ? 0 : (FR < tm ? FR : -1);

  // ---- phase 1: general tiles (band products, masks) ------------------------
  auto phase1 = [&](auto twok) {
  // path of each position term for a general tile
  auto modes_of = [&](int t, int& p2c_mode, int& p2c_which, int& c2p_mode, float& a_off) {
    const int k_lo = t * BN, k_hi = min(t * BN + BN, ext) - 1;
    p2c_mode = TERM_OFF;
    p2c_which = 0;   // which: 0 top row, 1 bottom row
    if (has_p2c) {
      if (k_lo - wg_qhi >= sat_top) { p2c_mode = TERM_CONST; p2c_which = 0; }
      else if (k_hi - wg_qlo <= sat_bot) { p2c_mode = TERM_CONST; p2c_which = 1; }
      else p2c_mode = TERM_BAND;
    }
    c2p_mode = TERM_OFF;
    a_off = 0.f;
    if (has_c2p && w_qlo <= w_qhi) {
      if (w_qlo - k_hi >= sat_top) { c2p_mode = TERM_CONST; a_off = a_top; }
      else if (w_qhi - k_lo <= sat_bot) { c2p_mode = TERM_CONST; a_off = a_bot; }
      else c2p_mode = TERM_BAND;
    }
  };

  constexpr int FB = (C::NBV + NW - 1) / NW;   // F blocks of one wave
  // this lane's half of a qr / kr row: base plus the row offset
  const unsigned char* qr_lane = QRg + (hoff + lh * C::HALF) * ES;
  const unsigned char* kr_lane = KRg + (hoff + lh * C::HALF) * ES;

  if (first_general >= 0) fetch(first_general * BN);
  else if (first_far >= 0) fetch(first_far * BN);
  for (int t = first_general; t >= 0; t = next_general(t)) {
    const int j0 = t * BN;
    const bool need_mask = j0 + BN > key_end;
    int p2c_mode, p2c_which, c2p_mode;
    float a_off;
    modes_of(t, p2c_mode, p2c_which, c2p_mode, a_off);

    const uint64_t kvalid = need_mask ? tile_valid(j0) : ~0ull;
    stage(Ks, Vt, cbuf, p2c_mode == TERM_CONST ? p2c_which : -1, kvalid);
    {
      const int tn = next_general(t);
      if (tn >= 0) {
        if (tn < tm) fetch_valid(tn * BN);
        else fetch(tn * BN);
      } else if (ES == 4 && first_far >= 0) {
        fetch_valid(first_far * BN);   // the register-staged far phase's first tile
      }
    }
    __syncthreads();  // K, V^T (and c_j) of this tile staged

    f32x16_t s[C::NKB];
    const bool far_tile = !need_mask && c2p_mode != TERM_BAND && p2c_mode != TERM_BAND;
    if (far_tile) {
      if (p2c_mode == TERM_CONST) far_scores(s, Ks, cbuf, std::true_type{});
      else far_scores(s, Ks, cbuf, std::false_type{});
    } else {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        // fp32 rows are wide: K is read from LDS per MFMA instead of held in
        // registers, and relative rows are fetched one block at a time
        const unsigned char* k_lds = Ks + ((kb * 32 + li) * C::KPITCH + lh * C::HALF) * ES;
        if (p2c_mode == TERM_BAND) {
          // F[jh][v] = k_(j0+32kb+jh) . qr[T(vmin + v)], v over BM+31 distances
          const int vmin = (j0 + 32 * kb) - (i0 + BM - 1);
#pragma unroll
          for (int x = 0; x < FB; ++x) {
            const int vb = wave + NW * x;
            if (vb < C::NBV) {
              uint4 rf[NU];
              load_half_row<NU>(rf, qr_lane + rel_off(vmin + vb * 32 + li, twok));
              const f32x16_t f = mma_chain_lds<T, NU, NC>(k_lds, rf, f32x16_t{});
#pragma unroll
              for (int r = 0; r < 16; ++r)
                Fw[(rr_of(r) + 4 * lh) * C::FWP + vb * 32 + li] = f[r];
            }
          }
        }
        if (c2p_mode == TERM_BAND) {
          // E[u][i] = kr[T(umin + u)] . q_i, u over the wave's 63 distances
          const int umin = i0w - (j0 + 32 * kb + 31);
#pragma unroll
          for (int ub = 0; ub < 2; ++ub) {
            uint4 rf[NU];
            load_half_row<NU>(rf, kr_lane + rel_off(umin + ub * 32 + li, twok));
            const f32x16_t e = mma_chain<T, NU, NC>(rf, qf, f32x16_t{});
#pragma unroll
            for (int r = 0; r < 16; ++r) Eww[(ub * 32 + rr_of(r) + 4 * lh) * 32 + li] = e[r];
          }
        }
        if (p2c_mode == TERM_BAND) __syncthreads();  // F complete

        f32x16_t acc = (p2c_mode == TERM_CONST) ? c_init(cbuf, kb) : f32x16_t{};
        acc = mma_chain_lds<T, NU, NC>(k_lds, qf, acc);
        if (c2p_mode == TERM_BAND) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] += e_base[(27 - rr_of(r)) * 32];
        }
        if (p2c_mode == TERM_BAND) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] += f_base[rr_of(r) * (C::FWP + 1)];
        }
        if (need_mask) {
          const uint32_t kv = (uint32_t)(kvalid >> (kb * 32 + 4 * lh));   // this lane's keys
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((kv >> rr_of(r)) & 1u)) acc[r] = NEG_INF;
        }
        s[kb] = acc;
        if (p2c_mode == TERM_BAND && kb + 1 < C::NKB) __syncthreads();  // F reused
      }
    }
    softmax_pv(s, a_off, vop_staged(v_base0));
    __syncthreads();  // tile buffers free for the next key tile
  }

  };
  if constexpr (ES == 4) {
    if (tw_ok) phase1(std::true_type{});
    else phase1(std::false_type{});
  }

  if constexpr (ES == 2) {
    // ---- K/V slots filled by direct-to-LDS loads (16-bit types) -------------
    // A slot holds a K tile and a V tile as dense [BN][D] rows. K rows are
    // stored with an XOR swizzle of their 16-byte units (conflict-free MFMA
    // operand reads); V rows as they are, read with the transposing LDS read
    // into the V^T operand.
    const uint32_t ring = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)smem;
    constexpr int DPW = C::DMA_PER_WAVE;
    constexpr int ROWB = C::UPR * 16;   // bytes of one slot row
    // source offsets of this wave's loads (unit order swizzled per row)
    uint32_t kdo[DPW], vdo[DPW];
#pragma unroll
    for (int x = 0; x < DPW; ++x) {
      const int u_lds = 64 * (wave * DPW + x) + lane;
      const int r = u_lds / C::UPR, pu = u_lds % C::UPR;
      kdo[x] = (uint32_t)((r * p.ld_k + hoff) * ES + 16 * (pu ^ C::swz_k(r)));
      vdo[x] = (uint32_t)((r * p.ld_v + hoff) * ES + 16 * (pu ^ C::swz_v(r)));
    }
    // load key tile t into the slot at LDS byte address slot_addr
    auto issue_tile = [&](int t, uint32_t slot_addr) {
      const int64_t j0 = (int64_t)t * BN;
      const unsigned char* kt = Kg + (base + j0) * p.ld_k * ES;
      const unsigned char* vt = Vg + (base + j0) * p.ld_v * ES;
      const uint32_t slot = slot_addr + 1024 * wave * DPW;
      if (j0 + BN <= ext) {
#pragma unroll
        for (int x = 0; x < DPW; ++x) dma16(slot + 1024 * x, kt, kdo[x]);
#pragma unroll
        for (int x = 0; x < DPW; ++x) dma16(slot + C::KT_BYTES + 1024 * x, vt, vdo[x]);
      } else {
        // the sequence ends inside the tile: rows past its end repeat its
        // last row (never read beyond it; those keys are masked)
        const int last = ext - 1 - (int)j0;
#pragma unroll
        for (int x = 0; x < DPW; ++x) {
          const int r = (64 * (wave * DPW + x) + lane) / C::UPR;
          const int back = r > last ? r - last : 0;
          dma16(slot + 1024 * x, kt, kdo[x] - (uint32_t)(back * p.ld_k * ES));
        }
#pragma unroll
        for (int x = 0; x < DPW; ++x) {
          const int r = (64 * (wave * DPW + x) + lane) / C::UPR;
          const int back = r > last ? r - last : 0;
          dma16(slot + C::KT_BYTES + 1024 * x, vt, vdo[x] - (uint32_t)(back * p.ld_v * ES));
        }
      }
    };

    // B operand of the c_j products (16x16x32 MFMA): column 0 is qr[top
    // row], column 1 qr[bottom row], the other columns zero
    typename Ty<T>::frag cq[D / 32];
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if ((lane & 15) < 2)
        x = ld16(Rrows + ((lane & 15) * D + 32 * m + 8 * (lane >> 4)) * ES);
      cq[m] = __builtin_bit_cast(typename Ty<T>::frag, x);
    }
    // c_j = k_j . qr[row] (which: 0 top, 1 bottom) of the 16 keys
    // 16g .. 16g+15 of a slot's K tile, stored at cdst[16g ..]
    auto c_group = [&](const unsigned char* ks, int g, int which, float* cdst) {
      const int r = 16 * g + (lane & 15);
      f32x4_t acc = f32x4_t{};
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        const int u = 4 * m + (lane >> 4);
        const auto a = __builtin_bit_cast(typename Ty<T>::frag,
                                          ld16(ks + r * ROWB + 16 * (u ^ C::swz_k(r))));
        acc = Ty<T>::mma16(a, cq[m], acc);
      }
      // lane l holds column l % 16 and keys 16g + 4*(l/16) + 0..3
      if ((lane & 15) == which)
        *reinterpret_cast<f32x4_t*>(cdst + 16 * g + 4 * (lane >> 4)) = acc;
    };

    // per-lane operand offsets inside a slot
    uint32_t kro[NU];   // K rows li (+32 kb), units lh*NU + x
#pragma unroll
    for (int x = 0; x < NU; ++x) kro[x] = li * ROWB + 16 * ((lh * NU + x) ^ C::swz_k(li));
    const int vg = lane >> 4, vt4 = lane & 15;
    const int vkey = 4 * (vg >> 1) + (vt4 >> 2);   // + 32 kb + 16 c + 8 h
    uint32_t vro[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int u = 4 * db + 2 * (vg & 1) + ((vt4 & 3) >> 1);
      vro[db] = vkey * ROWB + 16 * (u ^ C::swz_v(vkey)) + 8 * (vt4 & 1);
    }
    // V^T operand of the P.V MFMA from the V tile at vs
    auto vop_slot = [&](const unsigned char* vs) {
      return [=](int kb, int c, int db) {
        const unsigned char* a0 = vs + vro[db] + (32 * kb + 16 * c) * ROWB;
        const uint2 lo = lds_tr16(a0), hi = lds_tr16(a0 + 8 * ROWB);
        return __builtin_bit_cast(typename Ty<T>::frag, make_uint4(lo.x, lo.y, hi.x, hi.y));
      };
    };
    // this lane's K operand (key li of block kb) from the K tile at ks
    auto k_operand = [&](const unsigned char* ks, int kb, uint4 (&kf)[NU]) {
#pragma unroll
      for (int x = 0; x < NU; ++x) kf[x] = ld16(ks + kro[x] + kb * 32 * ROWB);
    };

    // ---- phase 1 (16-bit types): general tiles ------------------------------
    // Tiles with band terms or masked keys. Tile t sits in slot t's parity;
    // the next general tile is loaded while it is computed. A tile is worked
    // through per 32-key half, each half with its own softmax and P.V. Every
    // band product is wave-private: per 32-key half, E[u][i] = kr[T(u)] . q_i over
    // the 63 distances u = i - j of the wave's queries and F[j][v] =
    // k_j . qr[T(v)] over the 63 distances v = j - i are formed by MFMA
    // (table rows gathered into the operands), stored in the wave's LDS
    // scratch and read back along the diagonal, so no wave waits for another
    // within a tile. A term that is saturated over all of a wave's pairs
    // takes the constant path (a_i, or c_j from the wave's own small MFMAs).
    // One barrier per tile, two when the tile holds masked keys.
    auto phase1g = [&](auto twok) {
      float* scr = reinterpret_cast<float*>(smem + C::OFF_SCR + wave * C::SCR_BYTES);
      float* cjw = reinterpret_cast<float*>(smem + C::OFF_CJW + wave * BN * 4);
      const float* e_rd = scr + (li + 4 - 4 * lh) * 32 + li;   // + (27 - rr) * 32
      constexpr int FP = C::FPITCH;
      const float* f_rd = scr + 4 * lh * (FP + 1) + 31 - li;   // + rr * (FP + 1)
      struct Modes { int c2p, p2c, which; float a_off; };
      // paths of the two terms over this wave's pairs with tile t
      auto wave_modes = [&](int t) {
        Modes m;
        m.c2p = TERM_OFF;
        m.p2c = TERM_OFF;
        m.which = 0;
        m.a_off = 0.f;
        if (w_qlo > w_qhi) return m;   // no query of this wave exists
        const int k_lo = t * BN, k_hi = min(t * BN + BN, ext) - 1;
        if (has_p2c) {
          if (k_lo - w_qhi >= sat_top) { m.p2c = TERM_CONST; m.which = 0; }
          else if (k_hi - w_qlo <= sat_bot) { m.p2c = TERM_CONST; m.which = 1; }
          else m.p2c = TERM_BAND;
        }
        if (has_c2p) {
          if (w_qlo - k_hi >= sat_top) { m.c2p = TERM_CONST; m.a_off = a_top; }
          else if (w_qhi - k_lo <= sat_bot) { m.c2p = TERM_CONST; m.a_off = a_bot; }
          else m.c2p = TERM_BAND;
        }
        return m;
      };
      // one value per wave: branches on it stay scalar
      auto uniform = [](Modes m) {
        m.c2p = __builtin_amdgcn_readfirstlane(m.c2p);
        m.p2c = __builtin_amdgcn_readfirstlane(m.p2c);
        m.which = __builtin_amdgcn_readfirstlane(m.which);
        return m;
      };
      // Table rows of the band operands: for half kb of tile t, E block ub
      // covers the distances u = umin + 32 ub + 0..31 and F block vb the
      // distances v = vmin + 32 vb + 0..31; lane li fetches row li of a block.
      // Adjacent 32-key halves (the two halves of a tile, or the last half
      // of a tile and the first of the next tile when that is the adjacent
      // one) share blocks: a half's E block 1 is the E block 0 of the half
      // before it (same rows and queries, so the product is kept in
      // registers, not recomputed) and its F block 0 uses that half's F
      // block-1 rows. Three register blocks hold the rows: rE the E block 0,
      // rF[kb] and rF[kb ^ 1] the F blocks 0 and 1 of half kb (so the F
      // block-1 rows of one half are already in place as the next half's
      // block 0). Each half fetches the next half's rows as soon as its own
      // products have read the buffers, a whole half ahead of their use.
      const unsigned char* krb = KRg + hoff * ES;   // this head's columns
      const unsigned char* qrb = QRg + hoff * ES;
      const uint32_t lhb = (uint32_t)(lh * C::HALF * ES);
      uint4 rE[NU], rF[2][NU];
      auto load_e = [&](int t, int kb, int ub, uint4 (&dst)[NU]) {
        const int umin = i0w - (t * BN + 32 * kb + 31);
        load_half_row<NU>(dst, krb + (rel_off(umin + 32 * ub + li, twok) + lhb));
      };
      // F products as 16x16x32 MFMAs (d <= 64: three quarters of the 32x32
      // work, the two 16x16 corners no pair reaches skipped) or as two 32x32
      // chains (d = 128, where the longer 16x16 chains measured slower).
      // 16x16 form: F rows in the B-operand layout, F block vb (32
      // distances) is two 16-distance blocks bb, lane l holding the row of
      // distance 16 bb + l % 16 and, for each of the D / 32 k-steps m, its
      // 16-byte unit 4 m + l / 16 (dst[KS16 bb + m])
      constexpr bool F16 = D <= 64;
      constexpr int KS16 = D / 32;
      static_assert(2 * KS16 == NU, "two 16-distance blocks fill an F buffer");
      auto load_f = [&](int t, int kb, int vb, uint4 (&dst)[NU]) {
        const int vmin = (t * BN + 32 * kb) - (i0w + 31);
        if constexpr (F16) {
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            const unsigned char* row = qrb + rel_off(vmin + 32 * vb + 16 * bb + (lane & 15), twok);
#pragma unroll
            for (int m = 0; m < KS16; ++m) dst[KS16 * bb + m] = ld16(row + 16 * (4 * m + (lane >> 4)));
          }
        } else {
          load_half_row<NU>(dst, qrb + (rel_off(vmin + 32 * vb + li, twok) + lhb));
        }
      };
      // E[u][i] (two 32-distance blocks) into the scratch, then added along
      // the diagonal; likewise F[j][v]. The scratch is rewritten only after
      // this wave's own reads of it: LDS serves one wave's accesses in order.
      auto add_e = [&](const f32x16_t& e0, const f32x16_t& e1, f32x16_t& acc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) scr[(rr_of(r) + 4 * lh) * 32 + li] = e0[r];
#pragma unroll
        for (int r = 0; r < 16; ++r) scr[(32 + rr_of(r) + 4 * lh) * 32 + li] = e1[r];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += e_rd[(27 - rr_of(r)) * 32];
      };
      // 32x32 form: F block vb into the scratch; then its diagonal added
      auto put_f = [&](const f32x16_t& f, int vb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) scr[(rr_of(r) + 4 * lh) * FP + 32 * vb + li] = f[r];
      };
      // 16x16 form: F[j][v] of key half kb: 16x16x32 products of key
      // sub-block sb (keys 16 sb + 0..15, A operand from the K tile) with the
      // 16-distance blocks b = sb .. sb + 2 its pairs reach (the half's F
      // blocks 0 and 1 hold b = 0, 1 and 2, 3), each stored in the scratch
      // as it completes
      auto f_products = [&](const unsigned char* ks, int kb, const uint4 (&fb0)[NU],
                            const uint4 (&fb1)[NU]) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int r = 32 * kb + 16 * sb + (lane & 15);
          typename Ty<T>::frag ka[KS16];
#pragma unroll
          for (int m = 0; m < KS16; ++m)
            ka[m] = __builtin_bit_cast(typename Ty<T>::frag,
                                       ld16(ks + r * ROWB + 16 * ((4 * m + (lane >> 4)) ^ C::swz_k(r))));
#pragma unroll
          for (int b = sb; b < sb + 3; ++b) {
            f32x4_t acc = f32x4_t{};
#pragma unroll
            for (int m = 0; m < KS16; ++m) {
              const uint4 bq = b < 2 ? fb0[KS16 * b + m] : fb1[KS16 * (b - 2) + m];
              acc = Ty<T>::mma16(ka[m], __builtin_bit_cast(typename Ty<T>::frag, bq), acc);
            }
            // lane l holds distance 16 b + l % 16 of keys 16 sb + 4 (l / 16) + 0..3
#pragma unroll
            for (int i = 0; i < 4; ++i) scr[(16 * sb + 4 * (lane >> 4) + i) * FP + 16 * b + (lane & 15)] = acc[i];
          }
        }
      };
      auto sum_f = [&](f32x16_t& acc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += f_rd[rr_of(r) * (FP + 1)];
      };

      int t = first_general;
      int par = 0;   // slot of tile t
      issue_tile(t, ring);
      Modes m = uniform(wave_modes(t));
      // rows of the first half
      if (m.c2p == TERM_BAND) load_e(t, 0, 0, rE);
      if (m.p2c == TERM_BAND) { load_f(t, 0, 0, rF[0]); load_f(t, 0, 1, rF[1]); }
      f32x16_t e_keep = f32x16_t{};   // E block 1 of the coming half, valid when ek
      bool ek = false;
      while (t >= 0) {
        const int tn = next_general(t);
        const int j0 = t * BN;
        const bool need_mask = j0 + BN > key_end;
        uint64_t kvalid = ~0ull;
        if (need_mask) {
          const int j = j0 + lane;
          bool ok = j < ext;
          if (!VARLEN && mrow && ok && j >= first_bad) ok = mrow[j] != 0;
          kvalid = (uint64_t)__ballot(ok);
        }
        wait_vm<0>();
        __syncthreads();  // tile t in its slot; the other slot is free
        const unsigned char* ks = smem + par * C::SLOT_BYTES;
        const unsigned char* vs = ks + C::KT_BYTES;
        if (kvalid != ~0ull) {
          // masked or missing keys: zero their V rows (their scores are -inf)
          for (int x = tid; x < BN * C::UPR; x += NT) {
            const int r = x / C::UPR;
            if (!((kvalid >> r) & 1ull))
              *reinterpret_cast<uint4*>(const_cast<unsigned char*>(vs) + 16 * x) = make_uint4(0, 0, 0, 0);
          }
          __syncthreads();
        }
        // the next general tile's K and V go to the other slot now, a whole
        // tile ahead of their use (the slot's last reader, the previous
        // tile, is past the barrier above); a wait for this tile's row
        // loads also waits for these older loads, which costs less than
        // exposing them at the next tile's start
        if (tn >= 0) issue_tile(tn, ring + (par ^ 1) * C::SLOT_BYTES);
        m = uniform(m);
        const Modes mn = uniform(tn >= 0 ? wave_modes(tn) : Modes{TERM_OFF, TERM_OFF, 0, 0.f});
        if (m.p2c == TERM_CONST) {
#pragma unroll
          for (int g = 0; g < BN / 16; ++g) c_group(ks, g, m.which, cjw);
        }
        auto q_k = [&](int kb, const uint4 (&kf)[NU]) {
          const f32x16_t c = (m.p2c == TERM_CONST) ? c_init(cjw, kb) : f32x16_t{};
          return mma_chain<T, NU, NC>(kf, qf, c);
        };
        auto mask_keys = [&](int kb, f32x16_t& acc) {
          if (kvalid != ~0ull) {
            const uint32_t kv = (uint32_t)(kvalid >> (kb * 32 + 4 * lh));   // this lane's keys
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (!((kv >> rr_of(r)) & 1u)) acc[r] = NEG_INF;
          }
        };
        static_assert(C::NKB == 2, "two key halves per tile");
        // One 32-key half kb of tile t: its scores (C2C, then the P2C band,
        // whose K operand dies before the E product, then the C2P band),
        // then its softmax and P.V. The next half is (t, 1) or (tn, 0).
        auto half = [&](auto kbc) {
          constexpr int kb = decltype(kbc)::value;
          const Modes nm = kb == 0 ? m : mn;
          const bool has_next = kb == 0 || tn >= 0;
          const int nt = kb == 0 ? t : tn;
          constexpr int nkb = kb ^ 1;
          const bool nadj = kb == 0 || tn == t + 1;
          const bool eb = m.c2p == TERM_BAND, fb = m.p2c == TERM_BAND;
          const bool neb = has_next && nm.c2p == TERM_BAND, nfb = has_next && nm.p2c == TERM_BAND;
          uint4 (&F0B)[NU] = rF[kb];       // this half's F block 0; the next half's block 1
          uint4 (&F1B)[NU] = rF[kb ^ 1];   // this half's F block 1; the next half's block 0
          uint4 kf[NU];
          k_operand(ks, kb, kf);
          f32x16_t acc = q_k(kb, kf);
          if (fb) {
            if constexpr (F16) {
              f_products(ks, kb, F0B, F1B);
              if (nfb) load_f(nt, nkb, 1, F0B);
              if (nfb && !nadj) load_f(nt, nkb, 0, F1B);
            } else {
              const f32x16_t f0 = mma_chain<T, NU, NC>(kf, F0B, f32x16_t{});
              if (nfb) load_f(nt, nkb, 1, F0B);
              const f32x16_t f1 = mma_chain<T, NU, NC>(kf, F1B, f32x16_t{});
              if (nfb && !nadj) load_f(nt, nkb, 0, F1B);
              put_f(f0, 0);
              put_f(f1, 1);
            }
            sum_f(acc);
          } else if (nfb) {
            load_f(nt, nkb, 1, F0B);
            load_f(nt, nkb, 0, F1B);
          }
          if (eb) {
            const f32x16_t e0 = mma_chain<T, NU, NC>(rE, qf, f32x16_t{});
            if (!ek) {
              // first half of a C2P band run: its E block 1 from its rows now
              load_e(t, kb, 1, rE);
              e_keep = mma_chain<T, NU, NC>(rE, qf, f32x16_t{});
            }
            if (neb) load_e(nt, nkb, 0, rE);
            add_e(e0, e_keep, acc);
            e_keep = e0;
          } else if (neb) {
            load_e(nt, nkb, 0, rE);
          }
          ek = eb && nadj && neb;
          mask_keys(kb, acc);
          softmax_pv_half(acc, kb, m.a_off, vop_slot(vs));
        };
        half(std::integral_constant<int, 0>{});
        half(std::integral_constant<int, 1>{});
        t = tn;
        m = mn;
        par ^= 1;
      }
      wait_vm<0>();
      __syncthreads();  // slots and scratch free for the far tiles
    };
    if (first_general >= 0) {
      if (tw_ok) phase1g(std::true_type{});
      else phase1g(std::false_type{});
    }

    // ---- phase 2 (16-bit types): far tiles through LDS rings ---------------
    // Far tiles 0..FL-1 and FR..tm-1 are numbered n = 0, 1, ...; K tiles pass
    // through a ring of 3 slots (tile n in slot n % 3) and V tiles through a
    // ring of 5 (slot n % 5), filled by direct-to-LDS loads issued three
    // tiles ahead and waited for two steps after they are issued; one
    // barrier per tile publishes them.
    // Two-stage pipeline: step n issues, in one block, the Q.K MFMAs of tile
    // n+1 and the P.V MFMAs of tile n-1 between tile n's exponentials, so
    // the matrix unit has work while the exponentials run.
    // On far tiles the P2C term is k_j . qr[row] with one saturated row per
    // side, so it joins the Q.K product, and the softmax scale joins it too:
    // the B operand is (q_i + qr[row]) * tau * log2(e) (formed in fp32,
    // rounded once to the element type; q_i * tau * log2(e) without P2C),
    // and the MFMA chain starts from a per-lane bias block holding
    // a_i tau log2(e) - m_run, so it yields the exponent of the softmax
    // weight directly: no per-score arithmetic precedes the exponential.
    const int nfar = FL + max(tm - FR, 0);
    if (nfar > 0) {
      const float tl2 = p.scale_log2;
      constexpr int KS = 3, VS = 5;   // ring slots
      static_assert((KS + VS) * C::KT_BYTES <= C::RING_BYTES, "rings exceed the ring region");
      auto kslot_of = [](int n) { return (uint32_t)n % KS; };   // n >= 0
      auto vslot_of = [](int n) { return (uint32_t)n % VS; };
      auto kslot = [&](int n) { return smem + kslot_of(n) * C::KT_BYTES; };
      auto vslot = [&](int n) { return smem + (KS + vslot_of(n)) * C::KT_BYTES; };
      // Tiles are issued in order n = 0, 1, ..., so their sources follow
      // running pointers: one tile apart, with a jump over the general
      // tiles [FL, FR) when the right-hand run starts.
      const int64_t kstep = (int64_t)BN * p.ld_k * ES, vstep = (int64_t)BN * p.ld_v * ES;
      const int64_t kjump = (int64_t)(FR - FL) * kstep, vjump = (int64_t)(FR - FL) * vstep;
      const unsigned char* kt_nx = Kg + base * p.ld_k * ES;
      const unsigned char* vt_nx = Vg + base * p.ld_v * ES;
      const uint32_t wring = (uint32_t)__builtin_amdgcn_readfirstlane((int)(ring + 1024 * wave * DPW));
      auto issue = [&](int n) {
        if (__builtin_expect(n == FL, 0)) { kt_nx += kjump; vt_nx += vjump; }
        const uint32_t ks = wring + kslot_of(n) * C::KT_BYTES;
        const uint32_t vs = wring + (KS + vslot_of(n)) * C::KT_BYTES;
#pragma unroll
        for (int x = 0; x < DPW; ++x) dma16(ks + 1024 * x, kt_nx, kdo[x]);
#pragma unroll
        for (int x = 0; x < DPW; ++x) dma16(vs + 1024 * x, vt_nx, vdo[x]);
        kt_nx += kstep;
        vt_nx += vstep;
      };
      // (q_i + qr[row]) tau log2(e) (which: 0 top row, 1 bottom row, -1 no
      // row) in this lane's layout
      auto q_scaled = [&](int which, uint4 (&dst)[NU]) {
        uint4 rf[NU];
        if (which >= 0) lds_half_row<NU>(rf, Rrows + which * D * ES + lh * C::HALF * ES);
#pragma unroll
        for (int x = 0; x < NU; ++x) {
          const auto a = __builtin_bit_cast(typename Ty<T>::frag, qf[x]);
          const auto b = __builtin_bit_cast(typename Ty<T>::frag, rf[x]);
          f32x8_t v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = ((float)a[e] + (which >= 0 ? (float)b[e] : 0.f)) * tl2;
          dst[x] = __builtin_bit_cast(uint4, Ty<T>::cvt8(v));
        }
      };
      // accumulator start of every score block: a_i tau log2(e) - m_run
      // (m_run taken as 0 before the first offset is set)
      float off_run = 0.f;
      f32x16_t bias;
      auto set_bias = [&] {
        const float b = off_run - (m_run == NEG_INF ? 0.f : m_run);
#pragma unroll
        for (int r = 0; r < 16; ++r) bias[r] = b;
      };

      // Scores of tile n from K rows kf; the two key blocks' MFMA chains are
      // interleaved, so no MFMA waits for the one issued just before it.
      auto scores_from = [&](const uint4 (&kf)[C::NKB][NU], const uint4 (&qop)[NU], f32x16_t (&s)[C::NKB]) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) s[kb] = bias;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
            s[kb] = Ty<T>::mma(frag_at<T, NU>(kf[kb], c), frag_at<T, NU>(qop, c), s[kb]);
      };
      auto scores = [&](int n, const uint4 (&qop)[NU], f32x16_t (&s)[C::NKB]) {
        const unsigned char* ks = kslot(n);
        uint4 kf[C::NKB][NU];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) k_operand(ks, kb, kf[kb]);
        scores_from(kf, qop, s);
      };
      // the same from global memory: the cold path of step n, whose K slot
      // already receives tile n+3
      auto scores_global = [&](int n, const uint4 (&qop)[NU], f32x16_t (&s)[C::NKB]) {
        const int64_t j0 = (int64_t)(n < FL ? n : FR + (n - FL)) * BN;
        uint4 kf[C::NKB][NU];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
          load_half_row<NU>(kf[kb], Kg + ((base + j0 + 32 * kb + li) * p.ld_k + hoff + lh * C::HALF) * ES);
        scores_from(kf, qop, s);
      };
      // P = exp2(s - sub) rounded to the element type, into pf; returns
      // this lane's sum of the rounded P (sub only on the cold path)
      auto exps = [&](f32x16_t (&s)[C::NKB], PFrag& pf, auto cold, float sub) -> float {
        float ps4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            f32x8_t e8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float x = s[kb][8 * c2 + e];
              if constexpr (decltype(cold)::value) x -= sub;
              e8[e] = __builtin_amdgcn_exp2f(x);
            }
            pf[kb][c2] = Ty<T>::cvt8(e8);
            const uint4 w = __builtin_bit_cast(uint4, pf[kb][c2]);
            ps4[0] = Ty<T>::sum2(w.x, ps4[0]);
            ps4[1] = Ty<T>::sum2(w.y, ps4[1]);
            ps4[2] = Ty<T>::sum2(w.z, ps4[2]);
            ps4[3] = Ty<T>::sum2(w.w, ps4[3]);
          }
        return (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      };
      // Step n: scores of tile n in s_cur (read from K slot n % 3 before the
      // barrier that ended step n-1, or before a barrier of their own),
      // P of tile n-1 in pf_prev (its
      // P.V is still due). Forms the scores of tile n+1 in s_nxt and P of
      // tile n in pf_cur, and accumulates P.V of tile n-1.
      // The offset m_run is raised only when a tile's maximum exceeds it by
      // more than 8; the exponentials are taken against the current offset
      // and their row-half sum (at most 32 * 2^8 when no raise is due)
      // detects a due raise or an overflow. That rare case, and a lane with
      // no offset yet, forms the tile's scores again, raises the offset and
      // redoes the exponentials. Returns true when it raised the offset: the
      // bias block is then out of date, and so are the scores of tile n+1.
      auto step = [&](int n, const uint4 (&qop)[NU], f32x16_t (&s_cur)[C::NKB],
                      f32x16_t (&s_nxt)[C::NKB], const PFrag& pf_prev, PFrag& pf_cur) -> bool {
        const bool more = n + 3 < nfar;
        if (more) issue(n + 3);   // K slot of tile n, V slot of tile n-2
        // unconditional, so the MFMAs share a block with the exponentials;
        // past the last tile of a run they read a slot whose result is not
        // used
        // d <= 64 (built with the max-ilp scheduler): tile n+1's K operand is
        // read from LDS first, ahead of a scheduling barrier, so the Q.K
        // MFMAs find it in registers; max-ilp would otherwise issue each
        // read just before its MFMA and expose the LDS latency there. The
        // group hints then spread the exponentials over the MFMAs: per MFMA
        // two exponentials and one other VALU instruction. (d = 128, built
        // with the default scheduler, ran 4-5% slower with both.)
        constexpr bool PIN_K = D <= 64;
        if constexpr (PIN_K) {
          uint4 kf_n[C::NKB][NU];
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) k_operand(kslot(n + 1), kb, kf_n[kb]);
          __builtin_amdgcn_sched_barrier(0);
          scores_from(kf_n, qop, s_nxt);
        } else {
          scores(n + 1, qop, s_nxt);
        }
        pv_acc(pf_prev, s_cur, vop_slot(vslot(n + VS - 1)));   // tile n-1
        float ps = exps(s_cur, pf_cur, std::false_type{}, 0.f);
        if constexpr (PIN_K) {
#pragma unroll
          for (int g = 0; g < 2 * C::NKB * NU; ++g) {   // the step's MFMA count
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);   // two transcendental
            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // one VALU
          }
        }
        bool raised = false;
        if (__builtin_expect(__any(!(ps <= 32.f * 256.f) || m_run == NEG_INF), 0)) {
          scores_global(n, qop, s_cur);
          float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
              mx4[0] = fmaxf(mx4[0], s_cur[kb][r]);
              mx4[1] = fmaxf(mx4[1], s_cur[kb][r + 1]);
              mx4[2] = fmaxf(mx4[2], s_cur[kb][r + 2]);
              mx4[3] = fmaxf(mx4[3], s_cur[kb][r + 3]);
            }
          const float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
          const float mxf = fmaxf(mx, wave_xor32(mx));   // relative to the current offset
          const float m_eff = m_run == NEG_INF ? 0.f : m_run;
          const bool raise = m_run == NEG_INF || mxf > 8.f;
          const float m_new = raise ? m_eff + mxf : m_run;
          // m_run == -inf: nothing accumulated yet, alpha = exp2(-inf) = 0;
          // o_acc already holds tile n-1's P.V, taken at the old offset
          const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
          l_part *= alpha;
#pragma unroll
          for (int x = 0; x < C::NDB; ++x) o_acc[x] *= alpha;
          const float delta = m_new - m_eff;   // 0 without a raise
          m_run = m_new;
          ps = exps(s_cur, pf_cur, std::true_type{}, delta);
          raised = __any(raise);
        }
        l_part += ps;
        // tile n+2, read from the next step on, has landed once at most the
        // loads of tile n+3 are in flight; after the barrier it is visible
        // and the K slot of tile n+1 and the V slot of tile n-1 are free
        if (more) wait_vm<2 * DPW>();
        else wait_vm<0>();
        __syncthreads();
        return raised;
      };
      // The P.V of tile n-1 is due at step n. Before the first far tile it
      // is a zero P against a zero-filled V slot (the slot of tile -1).
      PFrag pfa, pfb;   // pfb: the pending P
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) pfb[kb][c2] = __builtin_bit_cast(typename Ty<T>::frag, make_uint4(0, 0, 0, 0));
      // tiles n0 .. n1-1 with B operand qop and C2P constant a_off. The bias
      // block is constant inside the inner loop; a raise of the offset
      // leaves it, and the outer loop forms the next tile's scores again
      // with the new bias.
      auto run = [&](int n0, int n1, const uint4 (&qop)[NU], float a_off) {
        off_run = a_off * tl2;
        int n = n0;
        while (n < n1) {
          set_bias();
          f32x16_t sa[C::NKB], sb[C::NKB];
          scores(n, qop, sa);
          // step n loads tile n+3 into the K slot just read: every wave's
          // reads of it come first
          __syncthreads();
          for (;;) {
            const bool r0 = step(n, qop, sa, sb, pfb, pfa);
            ++n;
            if (r0 || n >= n1) {
#pragma unroll
              for (int kb = 0; kb < C::NKB; ++kb) {
                pfb[kb][0] = pfa[kb][0];
                pfb[kb][1] = pfa[kb][1];
              }
              break;
            }
            const bool r1 = step(n, qop, sb, sa, pfa, pfb);
            ++n;
            if (r1 || n >= n1) break;
          }
        }
      };

      const int npre = min(nfar, 3);
      for (int n = 0; n < npre; ++n) issue(n);
      {
        // zero V slot VS-1, the slot of tile -1 (written by tile VS-1, issued
        // after the first step's barrier)
        unsigned char* z = smem + (KS + VS - 1) * C::KT_BYTES;
        for (int x = tid; x < C::KT_BYTES / 16; x += NT)
          *reinterpret_cast<uint4*>(z + 16 * x) = make_uint4(0, 0, 0, 0);
      }
      wait_vm<0>();
      __syncthreads();  // tiles 0 .. npre-1 in LDS, V slot of tile -1 zero
      const float a_left = has_c2p ? a_top : 0.f, a_right = has_c2p ? a_bot : 0.f;
      uint4 qop[NU];
      // keys left of the queries read the bottom qr row, keys right the top
      q_scaled(has_p2c ? 1 : -1, qop);
      run(0, FL, qop, a_left);
      if (has_p2c) q_scaled(0, qop);
      run(FL, nfar, qop, a_right);
      // the last tile's P.V
      f32x16_t unused[C::NKB];
      pv_acc(pfb, unused, vop_slot(vslot(nfar - 1)));
    }
  }

  // ---- phase 2 (fp32): far tiles, double-buffered through registers --------
  if (ES == 4 && first_far >= 0) {
    // which qr row the constant P2C term reads, and the C2P offset, per side
    auto p2c_row_of = [&](int t) { return has_p2c ? (t < FL ? 1 : 0) : -1; };
    int t = first_far;
    stage(Ks, Vt, cbuf, p2c_row_of(t), ~0ull);
    int tn = next_far(t);
    if (tn >= 0) fetch_valid(tn * BN);
    __syncthreads();
    int b = 0;
    while (t >= 0) {
      const int tnn = tn >= 0 ? next_far(tn) : -1;
      if (tn >= 0) {
        // the other buffer was last read by the previous tile, which every
        // wave has finished (barrier at the end of the previous iteration)
        if (b) stage(Ks, Vt, cbuf, p2c_row_of(tn), ~0ull);
        else stage(Ks1, Vt1, cbuf1, p2c_row_of(tn), ~0ull);
        if (tnn >= 0) fetch_valid(tnn * BN);
      }
      const float a_off = has_c2p ? (t < FL ? a_top : a_bot) : 0.f;
      f32x16_t s[C::NKB];
      if (has_p2c) far_scores(s, b ? Ks1 : Ks, b ? cbuf1 : cbuf, std::true_type{});
      else far_scores(s, b ? Ks1 : Ks, b ? cbuf1 : cbuf, std::false_type{});
      softmax_pv(s, a_off, vop_staged(b ? v_base1 : v_base0));
      __syncthreads();  // next tile staged; this tile's buffer free
      t = tn;
      tn = tnn;
      b ^= 1;
    }
  }

  // ---- epilogue: normalise, zero padded rows, store ----------------------
  {
    const float l_tot = l_part + wave_xor32(l_part);
    const int qi = i0w + li;
    bool row_ok = qi < ext && l_tot > 0.f;
    if (!VARLEN && mrow && qi < ext) row_ok = row_ok && mrow[qi] != 0;
    const float inv = row_ok ? 1.f / l_tot : 0.f;
    // log of the row's sum of exp(tau S): the exponentials were taken as
    // exp2(tau log2(e) S - m_run), so it is ln 2 (m_run + log2 l)
    if (p.lse && lh == 0 && qi < row_limit)
      p.lse[(base + qi) * p.H + head] = row_ok ? (m_run + log2f(l_tot)) * 0.6931471805599453f : NEG_INF;
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

// one work item per workgroup
template <class T, int D, int BN, int NW, bool VARLEN>
__global__ __launch_bounds__(64 * NW, (Cfg<T, D, BN, NW>::WG_PER_CU))
void dattn_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg<T, D, BN, NW>::LDS_BYTES];
  fwd_item<T, D, BN, NW, VARLEN>(p, blockIdx.x, smem);
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
  // Short padded batches with a mask may hold many query tiles with no valid
  // query (heavy right padding). Their items are ordered query tile first,
  // so the workgroups dispatched first hold the valid tiles and the
  // zero-only ones run behind them.
  p.qt_major = (!varlen && p.mask && p.L <= kShortPadded) ? 1 : 0;
  if (varlen)
    hipLaunchKernelGGL((dattn_fwd_kernel<T, D, BN, NW, true>), dim3((unsigned)n_work), dim3(C::NT), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((dattn_fwd_kernel<T, D, BN, NW, false>), dim3((unsigned)n_work), dim3(C::NT), 0,
                       stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Tile dispatch: 32 NW queries per workgroup, 64-key tiles (32 for fp32 at
// d = 128). A sweep of NW in {2, 4, 8} over the benchmark shapes
// (tune_tiles.py; 16-bit types) found NW = 4 fastest everywhere except
// packed batches of short sequences, where 64-query tiles leave fewer rows
// of a tile empty. Building with -DDATTN_NW_D32=n (D64, D128) fixes the wave
// count of the 16-bit instances for every length: the sweep's variants.
#if defined(DATTN_NW_D32) || defined(DATTN_NW_D64) || defined(DATTN_NW_D128)
constexpr bool kNwForced = true;
#else
constexpr bool kNwForced = false;
#endif
#ifndef DATTN_NW_D32
#define DATTN_NW_D32 4
#endif
#ifndef DATTN_NW_D64
#define DATTN_NW_D64 4
#endif
#ifndef DATTN_NW_D128
#define DATTN_NW_D128 4
#endif
constexpr int kShortPackedLen = 128;   // packed, max_seqlen up to this: 64-query tiles

// The fp16/bf16 d = 128 instances live in a unit of their own
// (dattn_fwd_d128.hip, which includes this file with the macro below set),
// compiled with another machine scheduler than the rest.
int launch_fwd_h16_d128(FwdParams& p, bool fp16, bool varlen, hipStream_t stream)
#ifdef DATTN_FWD_H16_D128_UNIT
{
  if (fp16) return launch_inst<TF16, 128, 64, DATTN_NW_D128>(p, varlen, stream);
  return launch_inst<TBF16, 128, 64, DATTN_NW_D128>(p, varlen, stream);
}
#else
;

template <class T>
int launch_dtype(FwdParams& p, int d, bool varlen, hipStream_t stream) {
  constexpr bool h16 = Ty<T>::ESIZE == 2;
  const bool short_packed = !kNwForced && varlen && p.max_seqlen <= kShortPackedLen;
  switch (d) {
    case 32:
      if constexpr (h16) {
        if (short_packed) return launch_inst<T, 32, 64, 2>(p, varlen, stream);
        return launch_inst<T, 32, 64, DATTN_NW_D32>(p, varlen, stream);
      } else {
        return launch_inst<T, 32, 64, 4>(p, varlen, stream);
      }
    case 64:
      if constexpr (h16) {
        if (short_packed) return launch_inst<T, 64, 64, 2>(p, varlen, stream);
        return launch_inst<T, 64, 64, DATTN_NW_D64>(p, varlen, stream);
      } else {
        return launch_inst<T, 64, 64, 4>(p, varlen, stream);
      }
    case 128:
      if constexpr (h16) return launch_fwd_h16_d128(p, std::is_same<T, TF16>::value, varlen, stream);
      else return launch_inst<T, 128, 32, 4>(p, varlen, stream);
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
#endif  // DATTN_FWD_H16_D128_UNIT

}  // namespace dattn
