// Projection of the relative-position embeddings into the per-head tables
// the disentangled scores read: qr = E Wq^T + bq and kr = E Wk^T + bk, with
// E the [n_rel, hidden] relative embeddings shared by the batch and
// nn.Linear-style weights ([H*d, hidden]). In DeBERTa-v2/v3, the models the
// DisentangledFlash README's "Attribution" section names, these are the
// attention layer's own query and key maps applied to the relative
// embeddings.
//
// One launch forms both tables. A workgroup owns a 64 x 64 output tile of
// one table (blockIdx.z: 0 = qr, 1 = kr) and each of its four waves a
// 32 x 32 block, accumulated by 32x32 MFMAs in fp32. The reduction runs in
// stages of 256 bytes of every row: the workgroup's 64 rows of E and of W
// for a stage go to LDS (double-buffered; the next stage is loaded into
// registers while the current one is multiplied), so each row is read from
// L2 once per tile rather than once per wave. Both operands keep the
// reduction dimension contiguous: within a 16-element chunk, lane half h
// supplies elements 8h .. 8h+7 of both, which pairs A and B elements of the
// same index. Rows and columns past the ends are read clamped and not
// stored; a partly full last stage is zero-filled. The bias is added and
// the result rounded once to the element type.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dattn_internal.h"

namespace dattn {

namespace {

typedef __bf16 rp_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 rp_f16x8 __attribute__((ext_vector_type(8)));
typedef float rp_f32x16 __attribute__((ext_vector_type(16)));

constexpr int RP_TILE = 64;    // output rows and columns of a workgroup
constexpr int RP_CHUNK = 16;   // reduction elements per MFMA step group
#ifndef RP_STAGE_BYTES
#define RP_STAGE_BYTES 256     // bytes of every row staged in LDS per step
#endif

struct RelProjParams {
  const unsigned char* E;
  int64_t ld_e;
  const unsigned char* W[2];
  int64_t ld_w;
  const unsigned char* bias[2];
  unsigned char* out[2];
  int64_t ld_out;
  int32_t n_rel, hidden, HD;
};

__device__ __forceinline__ uint4 ldg16(const unsigned char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int DT> struct RP;   // DT: element type code of the ABI
template <> struct RP<0> {     // fp32: eight 32x32x2 steps per 16-element chunk
  static constexpr int ES = 4;
  static constexpr int U = 2;  // 16-byte units per lane per chunk
  __device__ static rp_f32x16 step(const uint4 (&a)[U], const uint4 (&b)[U], rp_f32x16 acc) {
    const float av[8] = {__builtin_bit_cast(float, a[0].x), __builtin_bit_cast(float, a[0].y),
                         __builtin_bit_cast(float, a[0].z), __builtin_bit_cast(float, a[0].w),
                         __builtin_bit_cast(float, a[1].x), __builtin_bit_cast(float, a[1].y),
                         __builtin_bit_cast(float, a[1].z), __builtin_bit_cast(float, a[1].w)};
    const float bv[8] = {__builtin_bit_cast(float, b[0].x), __builtin_bit_cast(float, b[0].y),
                         __builtin_bit_cast(float, b[0].z), __builtin_bit_cast(float, b[0].w),
                         __builtin_bit_cast(float, b[1].x), __builtin_bit_cast(float, b[1].y),
                         __builtin_bit_cast(float, b[1].z), __builtin_bit_cast(float, b[1].w)};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s], bv[s], acc, 0, 0, 0);
    return acc;
  }
  __device__ static float load(const unsigned char* p) { return *reinterpret_cast<const float*>(p); }
  __device__ static void store(unsigned char* p, float x) { *reinterpret_cast<float*>(p) = x; }
};
template <> struct RP<1> {     // fp16: one 32x32x16 step per chunk
  static constexpr int ES = 2;
  static constexpr int U = 1;
  __device__ static rp_f32x16 step(const uint4 (&a)[U], const uint4 (&b)[U], rp_f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(rp_f16x8, a[0]),
                                                  __builtin_bit_cast(rp_f16x8, b[0]), acc, 0, 0, 0);
  }
  __device__ static float load(const unsigned char* p) {
    return (float)*reinterpret_cast<const _Float16*>(p);
  }
  __device__ static void store(unsigned char* p, float x) { *reinterpret_cast<_Float16*>(p) = (_Float16)x; }
};
template <> struct RP<2> {     // bf16: one 32x32x16 step per chunk
  static constexpr int ES = 2;
  static constexpr int U = 1;
  __device__ static rp_f32x16 step(const uint4 (&a)[U], const uint4 (&b)[U], rp_f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(rp_bf16x8, a[0]),
                                                   __builtin_bit_cast(rp_bf16x8, b[0]), acc, 0, 0, 0);
  }
  __device__ static float load(const unsigned char* p) {
    return (float)*reinterpret_cast<const __bf16*>(p);
  }
  __device__ static void store(unsigned char* p, float x) { *reinterpret_cast<__bf16*>(p) = (__bf16)x; }
};

template <int DT>
__global__ __launch_bounds__(256) void rel_proj_kernel(const RelProjParams p) {
  typedef RP<DT> R;
  constexpr int ES = R::ES, U = R::U;
  constexpr int SB = RP_STAGE_BYTES;      // bytes of a row per stage
  constexpr int UPR = SB / 16;            // 16-byte units of a row per stage
  constexpr int UPT = SB / 64;            // units per thread per tile and stage
  constexpr int CB = RP_CHUNK * ES;       // bytes of a 16-element chunk
  constexpr int PITCH = SB + 16;          // LDS row pitch (bytes)
  static_assert(SB % CB == 0 && UPT >= 1, "stage size");
  __shared__ __align__(16) unsigned char lds[2][2][RP_TILE * PITCH];   // [buffer][E, W][row]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int wr = wave >> 1, wc = wave & 1;   // this wave's 32 x 32 block of the tile
  const int z = blockIdx.z;
  const int r0 = blockIdx.y * RP_TILE, o0 = blockIdx.x * RP_TILE;
  // loader: unit x = t + 256 j (j < UPT) of a tile is 16-byte unit x % UPR of
  // row x / UPR; both tiles, rows read clamped into the arrays
  const unsigned char* ga[UPT];
  const unsigned char* gb[UPT];
  int lrow[UPT], lu[UPT];
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int x = tid + 256 * j;
    lrow[j] = x / UPR;
    lu[j] = x % UPR;
    ga[j] = p.E + (int64_t)min(r0 + lrow[j], p.n_rel - 1) * p.ld_e * ES;
    gb[j] = p.W[z] + (int64_t)min(o0 + lrow[j], p.HD - 1) * p.ld_w * ES;
  }
  const int64_t row_bytes = (int64_t)p.hidden * ES;
  const int nst = (int)((row_bytes + SB - 1) / SB);
  uint4 va[UPT], vb[UPT];
  auto fetch = [&](int st) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int64_t off = (int64_t)st * SB + 16 * lu[j];
      const bool in = off < row_bytes;   // the last stage may be partly full
      va[j] = in ? ldg16(ga[j] + off) : make_uint4(0, 0, 0, 0);
      vb[j] = in ? ldg16(gb[j] + off) : make_uint4(0, 0, 0, 0);
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      *reinterpret_cast<uint4*>(&lds[buf][0][lrow[j] * PITCH + 16 * lu[j]]) = va[j];
      *reinterpret_cast<uint4*>(&lds[buf][1][lrow[j] * PITCH + 16 * lu[j]]) = vb[j];
    }
  };
  rp_f32x16 acc = {};
  fetch(0);
  put(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) fetch(st + 1);
    const unsigned char* la = &lds[buf][0][(32 * wr + li) * PITCH + 8 * lh * ES];
    const unsigned char* lb = &lds[buf][1][(32 * wc + li) * PITCH + 8 * lh * ES];
#pragma unroll
    for (int c = 0; c < SB / CB; ++c) {
      uint4 a[U], b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a[u] = *reinterpret_cast<const uint4*>(la + c * CB + 16 * u);
        b[u] = *reinterpret_cast<const uint4*>(lb + c * CB + 16 * u);
      }
      acc = R::step(a, b, acc);
    }
    if (st + 1 < nst) put(buf ^ 1);
    __syncthreads();   // the next stage is in; this one may be overwritten
  }

  // lane: output column; register r: row 8 (r / 4) + 4 lh + r % 4 of the block
  const int o = o0 + 32 * wc + li;
  if (o >= p.HD) return;
  const float bias = p.bias[z] ? R::load(p.bias[z] + (int64_t)o * ES) : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + 32 * wr + 8 * (r >> 2) + 4 * lh + (r & 3);
    if (row < p.n_rel) R::store(p.out[z] + ((int64_t)row * p.ld_out + o) * ES, acc[r] + bias);
  }
}

}  // namespace

int launch_rel_proj(const void* E, int64_t ld_e, const void* Wq, const void* Wk, int64_t ld_w,
                    const void* bq, const void* bk, void* qr, void* kr, int64_t ld_out,
                    int32_t n_rel, int32_t hidden, int32_t HD, int dtype, hipStream_t stream) {
  RelProjParams p;
  p.E = static_cast<const unsigned char*>(E);
  p.ld_e = ld_e;
  p.W[0] = static_cast<const unsigned char*>(Wq);
  p.W[1] = static_cast<const unsigned char*>(Wk);
  p.ld_w = ld_w;
  p.bias[0] = static_cast<const unsigned char*>(bq);
  p.bias[1] = static_cast<const unsigned char*>(bk);
  p.out[0] = static_cast<unsigned char*>(qr);
  p.out[1] = static_cast<unsigned char*>(kr);
  p.ld_out = ld_out;
  p.n_rel = n_rel;
  p.hidden = hidden;
  p.HD = HD;
  const dim3 grid((HD + RP_TILE - 1) / RP_TILE, (n_rel + RP_TILE - 1) / RP_TILE, 2);
  const dim3 block(256);
  if (dtype == 0) hipLaunchKernelGGL(rel_proj_kernel<0>, grid, block, 0, stream, p);
  else if (dtype == 1) hipLaunchKernelGGL(rel_proj_kernel<1>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(rel_proj_kernel<2>, grid, block, 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace dattn
