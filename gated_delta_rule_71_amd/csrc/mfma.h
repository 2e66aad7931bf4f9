// CDNA4 (gfx950) matrix-core helpers for 16x16 output tiles.
//
// Output tile layout (all 16x16 MFMAs): lane l, accumulator element i holds
// D[4 * (l / 16) + i][l % 16].
//
// Operand fragments: lane l supplies row (A) or column (B) l % 16 and eight
// (or four) values along K.  The hardware pairs A's slot (l / 16, j) with B's
// slot (l / 16, j) for the same k, so any bijection between (lane group, slot)
// and k gives the same product as long as A and B use the same one.  Two
// bijections are used here:
//   standard : lane group g, slot j  <->  k = 8g + j              (K = 32 block)
//   tile pair: lane group g, slot j  <->  k = 4g + j       (j < 4)
//                                         16 + 4g + j - 4  (j >= 4)
// The tile-pair order is exactly what the accumulators of two stacked 16-row
// output tiles hold in one lane, so an accumulated result can feed the next
// product as its B operand without leaving registers.
#pragma once
#include <hip/hip_runtime.h>

namespace gdr {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <typename OT>
struct Mma;

// bf16 operands, fp32 accumulate: 16x16x32 (K = 32 per instruction) and 16x16x16.
template <>
struct Mma<__bf16> {
  using F8 = bf16x8;
  using F4 = bf16x4;
  __device__ __forceinline__ static f32x4 mma8(const F8& a, const F8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4 mma4(const F4& a, const F4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
};

// fp32 operands: a K = 32 (or 16) block is 8 (or 4) 16x16x4 instructions; instruction
// j takes slot j of every lane, so the (lane group, slot) -> k bijection is unchanged.
template <>
struct Mma<float> {
  using F8 = f32x8;
  using F4 = f32x4;
  __device__ __forceinline__ static f32x4 mma8(const F8& a, const F8& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
  __device__ __forceinline__ static f32x4 mma4(const F4& a, const F4& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
};

template <typename OT>
__device__ __forceinline__ OT to_ot(float f) {
  return static_cast<OT>(f);
}

// 8 consecutive elements of an LDS row (16-byte aligned for bf16, 32 for fp32).
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::F8 lds_load8(const OT* p) {
  return *reinterpret_cast<const typename Mma<OT>::F8*>(p);
}
// 4 consecutive elements.
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::F4 lds_load4(const OT* p) {
  return *reinterpret_cast<const typename Mma<OT>::F4*>(p);
}

// A or B fragment in tile-pair order from a row of an LDS array: k0 is the start of the
// 32-wide k block, g the lane group.  Elements beyond `kmax` read as zero.
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::F8 lds_pair_frag(const OT* row, int k0, int g,
                                                              int kmax) {
  typename Mma<OT>::F8 f;
  const int ka = k0 + 4 * g, kb = k0 + 16 + 4 * g;
  typename Mma<OT>::F4 lo, hi;
  if (ka < kmax) {
    lo = lds_load4(row + ka);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) lo[j] = OT(0.f);
  }
  if (kb < kmax) {
    hi = lds_load4(row + kb);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) hi[j] = OT(0.f);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = lo[j];
    f[4 + j] = hi[j];
  }
  return f;
}

// Standard-order fragment (k = k0 + 8g + j); elements beyond kmax read as zero.
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::F8 lds_std_frag(const OT* row, int k0, int g,
                                                             int kmax) {
  const int k = k0 + 8 * g;
  if (k < kmax) return lds_load8(row + k);
  typename Mma<OT>::F8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = OT(0.f);
  return f;
}

// The same two loads with the range known at compile time: when KMAX is a multiple of 32
// every lane's k lies in range and the loads are unconditional (no branch per fragment).
template <int KMAX, typename OT>
__device__ __forceinline__ typename Mma<OT>::F8 lds_pair_frag_k(const OT* row, int k0, int g) {
  if constexpr (KMAX % 32 == 0) {
    typename Mma<OT>::F8 f;
    const typename Mma<OT>::F4 lo = lds_load4(row + k0 + 4 * g), hi = lds_load4(row + k0 + 16 + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = lo[j];
      f[4 + j] = hi[j];
    }
    return f;
  } else {
    return lds_pair_frag(row, k0, g, KMAX);
  }
}
template <int KMAX, typename OT>
__device__ __forceinline__ typename Mma<OT>::F8 lds_std_frag_k(const OT* row, int k0, int g) {
  if constexpr (KMAX % 32 == 0) {
    return lds_load8(row + k0 + 8 * g);
  } else {
    return lds_std_frag(row, k0, g, KMAX);
  }
}

// B fragment (tile-pair order) from two stacked accumulator tiles.
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::F8 acc_pair_frag(const f32x4& lo, const f32x4& hi) {
  typename Mma<OT>::F8 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = to_ot<OT>(lo[j]);
    f[4 + j] = to_ot<OT>(hi[j]);
  }
  return f;
}

// K = 16 fragment (k = 4g + j) from one accumulator tile.
template <typename OT>
__device__ __forceinline__ typename Mma<OT>::F4 acc_frag4(const f32x4& t) {
  typename Mma<OT>::F4 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = to_ot<OT>(t[j]);
  return f;
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

}  // namespace gdr
