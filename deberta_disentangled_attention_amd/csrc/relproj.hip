// Projection of the relative-position embeddings into the per-head tables
// the disentangled scores read: qr = E Wq^T + bq and kr = E Wk^T + bk, with
// E the [n_rel, hidden] relative embeddings shared by the batch and
// nn.Linear-style weights ([H*d, hidden]). In DeBERTa-v2/v3, the models the
// DisentangledFlash README's "Attribution" section names, these are the
// attention layer's own query and key maps applied to the relative
// embeddings.
//
// One launch forms both tables. A workgroup owns a 32 x 32 output block of
// one table (blockIdx.z: 0 = qr, 1 = kr); its four waves split the hidden
// dimension (wave w takes 16-element chunks w, w+4, ...), each accumulating
// a 32x32 MFMA product in fp32, and the partial blocks are summed through
// LDS. The problem is small (a v3-base table is 2 x 0.6 GFLOP), so the split
// is what keeps enough loads in flight: each wave loads its next group of
// chunks while it multiplies the current one. Both operands keep the
// reduction dimension contiguous in memory, so every lane reads its operand
// fragment straight from global memory as 16-byte units: within a chunk,
// lane half h supplies elements 8h .. 8h+7 for both operands, which pairs A
// and B elements of the same index. Rows and columns past the ends are read
// clamped and not stored. The bias is added and the result rounded once to
// the element type.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dattn_internal.h"

namespace dattn {

namespace {

typedef __bf16 rp_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 rp_f16x8 __attribute__((ext_vector_type(8)));
typedef float rp_f32x16 __attribute__((ext_vector_type(16)));

constexpr int RP_TILE = 32;
constexpr int RP_CHUNK = 16;   // reduction elements per step
#ifndef RP_UNROLL_STEPS
#define RP_UNROLL_STEPS 4
#endif
constexpr int RP_UNROLL = RP_UNROLL_STEPS;   // steps whose loads are issued together
constexpr int RP_WAVES = 4;    // waves splitting the reduction

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
__global__ __launch_bounds__(64 * RP_WAVES) void rel_proj_kernel(const RelProjParams p) {
  typedef RP<DT> R;
  constexpr int ES = R::ES, U = R::U;
  __shared__ float part[RP_WAVES - 1][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int z = blockIdx.z;
  const int r0 = blockIdx.y * RP_TILE, o0 = blockIdx.x * RP_TILE;
  // this lane's operand rows, clamped into the arrays
  const int ra = min(r0 + li, p.n_rel - 1), oa = min(o0 + li, p.HD - 1);
  const unsigned char* ea = p.E + (int64_t)ra * p.ld_e * ES + 8 * lh * ES;
  const unsigned char* wa = p.W[z] + (int64_t)oa * p.ld_w * ES + 8 * lh * ES;

  const int nchunk = p.hidden / RP_CHUNK;
  // group g of this wave: chunks (g * RP_UNROLL + s) * RP_WAVES + wave
  const int per_group = RP_UNROLL * RP_WAVES;
  const int ngroups = (nchunk + per_group - 1) / per_group;
  typedef uint4 Ops[RP_UNROLL][U];
  auto load_group = [&](int g, Ops& a, Ops& b) {
#pragma unroll
    for (int s = 0; s < RP_UNROLL; ++s) {
      const int c = (g * RP_UNROLL + s) * RP_WAVES + wave;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c < nchunk) {
          a[s][u] = ldg16(ea + ((int64_t)c * RP_CHUNK) * ES + 16 * u);
          b[s][u] = ldg16(wa + ((int64_t)c * RP_CHUNK) * ES + 16 * u);
        } else {
          a[s][u] = make_uint4(0, 0, 0, 0);
          b[s][u] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  rp_f32x16 acc = {};
  auto mult = [&](const Ops& a, const Ops& b) {
#pragma unroll
    for (int s = 0; s < RP_UNROLL; ++s) acc = R::step(a[s], b[s], acc);
  };
  Ops a0, b0, a1, b1;
  if (ngroups > 0) load_group(0, a0, b0);
  for (int g = 0; g < ngroups; g += 2) {
    if (g + 1 < ngroups) load_group(g + 1, a1, b1);
    mult(a0, b0);
    if (g + 2 < ngroups) load_group(g + 2, a0, b0);
    if (g + 1 < ngroups) mult(a1, b1);
  }

  // partial blocks of waves 1.. through LDS; wave 0 sums and stores
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < RP_WAVES - 1; ++w)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += part[w][r][lane];
  // lane: output column o0 + li; register r: row r0 + 8 (r / 4) + 4 lh + r % 4
  const int o = o0 + li;
  if (o >= p.HD) return;
  const float bias = p.bias[z] ? R::load(p.bias[z] + (int64_t)o * ES) : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + 8 * (r >> 2) + 4 * lh + (r & 3);
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
  const dim3 block(64 * RP_WAVES);
  if (dtype == 0) hipLaunchKernelGGL(rel_proj_kernel<0>, grid, block, 0, stream, p);
  else if (dtype == 1) hipLaunchKernelGGL(rel_proj_kernel<1>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(rel_proj_kernel<2>, grid, block, 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace dattn
