// Device-side building blocks shared by the forward and backward kernels
// of the disentangled attention (MI355X, gfx950): element types and their
// MFMA instructions, fragment helpers, wave reductions and small LDS/global
// access helpers.
#ifndef DATTN_DEVICE_H
#define DATTN_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));


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
  __device__ static __forceinline__ f32x4_t mma16(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag cvt8(f32x8_t x) {
    return __builtin_convertvector(x, bf16x8_t);
  }
  // acc + the two bf16 halves of w
  __device__ static __forceinline__ float sum2(uint32_t w, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w),
                                           __builtin_bit_cast(b2, 0x3f803f80u), acc, false);
  }
};

template <> struct Ty<TF16> {
  static constexpr int ESIZE = 2;
  static constexpr int LANE_K = 8;
  typedef f16x8_t frag;
  __device__ static __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4_t mma16(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag cvt8(f32x8_t x) {
    return __builtin_convertvector(x, f16x8_t);
  }
  // acc + the two fp16 halves of w
  __device__ static __forceinline__ float sum2(uint32_t w, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), __builtin_bit_cast(h2, 0x3c003c00u), acc,
                                  false);
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

// acc += A . B^T where A's half-row fragment is read from LDS a few units at
// a time (keeps few registers live for wide fp32 rows)
template <class T, int NU, int NC>
__device__ __forceinline__ f32x16_t mma_chain_lds(const unsigned char* a_lds, const uint4 (&b)[NU],
                                                  f32x16_t acc) {
  constexpr int CPU = NC / NU;   // MFMAs per 16-byte unit
#pragma unroll
  for (int x = 0; x < NU; ++x) {
    const uint4 a = *reinterpret_cast<const uint4*>(a_lds + 16 * x);
#pragma unroll
    for (int c = 0; c < CPU; ++c) {
      uint4 one[1] = {a};
      uint4 bb[1] = {b[x]};
      acc = Ty<T>::mma(frag_at<T, 1>(one, c), frag_at<T, 1>(bb, c), acc);
    }
  }
  return acc;
}

template <int NU>
__device__ __forceinline__ void load_half_row(uint4 (&u)[NU], const unsigned char* p) {
#pragma unroll
  for (int x = 0; x < NU; ++x) u[x] = ld16(p + 16 * x);
}

template <int NU>
__device__ __forceinline__ void lds_half_row(uint4 (&u)[NU], const unsigned char* p) {
#pragma unroll
  for (int x = 0; x < NU; ++x) u[x] = *reinterpret_cast<const uint4*>(p + 16 * x);
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32); }

// Wave-wide integer minimum / maximum by DPP (no LDS traffic): shifts by
// 1, 2, 4 and 8 lanes within each 16-lane row leave the row's result in its
// lane 15; row_bcast:15 then carries rows 0 and 2 into rows 1 and 3, and
// row_bcast:31 carries row 1 into rows 2 and 3, so lane 63 holds the
// wave's result. Lanes whose DPP source is absent keep the identity. The
// result is wave-uniform (a scalar register).
template <bool MAX>
__device__ __forceinline__ int wave_reduce_i(int x) {
  constexpr int ID = MAX ? (-2147483647 - 1) : 2147483647;
  auto op = [](int a, int b) { return MAX ? max(a, b) : min(a, b); };
  x = op(x, __builtin_amdgcn_update_dpp(ID, x, 0x111, 0xf, 0xf, false));   // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(ID, x, 0x112, 0xf, 0xf, false));   // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(ID, x, 0x114, 0xf, 0xf, false));   // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(ID, x, 0x118, 0xf, 0xf, false));   // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(ID, x, 0x142, 0xa, 0xf, false));   // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(ID, x, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ int wave_min_i(int x) { return wave_reduce_i<false>(x); }
__device__ __forceinline__ int wave_max_i(int x) { return wave_reduce_i<true>(x); }

// Direct-to-LDS load (global_load_lds_dwordx4): lane i's 16 bytes at
// gbase + voff are written to LDS byte address lds + 16 i. The data bypasses
// the registers; completion is tracked by this wave's vmcnt. Inline assembly
// rather than the compiler's builtin for this load: with the builtin, the
// compiler waits for every outstanding direct load (vmcnt(0)) before any LDS
// read it cannot prove disjoint, which would serialise the ring below; the
// explicit waits (wait_vm) keep the newest loads in flight instead. m0 is
// set here and declared clobbered; nothing else in these kernels uses it.
__device__ __forceinline__ void dma16(uint32_t lds, const void* gbase, uint32_t voff) {
  const uint64_t g = (uint64_t)(size_t)gbase;
  const uint64_t gu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(g >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)g);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(gu) : "memory", "m0");
}

// wait until at most N of this wave's vector-memory operations are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations (not for its outstanding global stores, which __syncthreads'
// full fence would wait for) and synchronises the workgroup.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16). In each group of 16 lanes, lane
// t names a 4-element chunk X_t; lane t receives X_(t/4 + 4e)[t % 4], e = 0..3.
__device__ __forceinline__ uint2 lds_tr16(const unsigned char* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  // every lane has a source lane in the patterns used here; bound_ctrl lets
  // the move fuse into the consuming add
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                0xf, 0xf, true));
}

// sum over each aligned group of N consecutive lanes (N = 4, 8, 16 or 32);
// every lane of a group receives the group's sum
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xb1>(x);                       // quad_perm [1,0,3,2]
  x += dpp<0x4e>(x);                       // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// dot product of two 16-byte units (8 bf16 / 8 fp16 / 4 fp32), fp32 accumulate
template <class T>
__device__ __forceinline__ float dot16(uint4 a, uint4 b) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (std::is_same<T, TBF16>::value) {
      typedef __bf16 b2 __attribute__((ext_vector_type(2)));
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, av[t]), __builtin_bit_cast(b2, bv[t]),
                                            acc, false);
    } else if constexpr (std::is_same<T, TF16>::value) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, av[t]), __builtin_bit_cast(h2, bv[t]), acc,
                                   false);
    } else {
      acc = fmaf(__builtin_bit_cast(float, av[t]), __builtin_bit_cast(float, bv[t]), acc);
    }
  }
  return acc;
}

// key offset (within a 32-key block) of accumulator register r in lane half 0
__device__ __forceinline__ constexpr int rr_of(int r) { return 8 * (r >> 2) + (r & 3); }

// Column of key k in a 16-bit V^T tile row. The P.V MFMA takes, in lane half
// h, the eight P values of registers 8c..8c+7 as its reduction elements
// 8h..8h+7; those are keys {16c + 4h + 0..3, 16c + 8 + 4h + 0..3}. Storing each
// group of 16 keys in the order 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 of the
// key swapped) makes the matching eight V^T elements contiguous.
__device__ __forceinline__ constexpr int v_pos(int k) {
  return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Smallest x in [0, n) with pred(x) true (pred monotone false -> true), or n.
// Every thread of the workgroup must call it; NT-way parallel search.
template <int NT, class Pred>
__device__ int block_first_true(int n, Pred pred, int* slot, int tid) {
  int lo = -1, hi = n;  // pred(lo) taken false, pred(hi) taken true
  while (hi - lo > 1) {
    const int span = hi - lo - 1;
    const int step = (span + NT - 1) / NT;
    if (tid == 0) *slot = NT;
    __syncthreads();
    const int x = lo + 1 + tid * step;
    if (x < hi && pred(x)) atomicMin(slot, tid);
    __syncthreads();
    const int k = *slot;
    __syncthreads();
    if (k == NT) {
      // every tested candidate is false: continue after the last one tested
      const int ncand = min(NT, (span + step - 1) / step);
      lo = lo + 1 + (ncand - 1) * step;
    } else {
      hi = lo + 1 + k * step;
      if (k > 0) lo = lo + 1 + (k - 1) * step;
    }
  }
  return hi;
}

}  // namespace dattn

#endif  // DATTN_DEVICE_H
