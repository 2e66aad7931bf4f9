// Shared device helpers for the gfx950 kernels: bf16 <-> fp32 and typed I/O.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// bf16 storage type as 16 raw bits; the arithmetic is always fp32.
struct bf16_t {
  uint16_t x;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename IO>
struct io_traits;

template <>
struct io_traits<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) {
    return bf16_to_f32(p[i].x);
  }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float f) {
    p[i].x = f32_to_bf16(f);
  }
};

template <>
struct io_traits<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float f) { p[i] = f; }
};

template <typename IO>
__device__ __forceinline__ float ld(const IO* p, int64_t i) {
  return io_traits<IO>::load(p, i);
}
template <typename IO>
__device__ __forceinline__ void st(IO* p, int64_t i, float f) {
  io_traits<IO>::store(p, i, f);
}

enum GateKind : int { kNone = 0, kScalar = 1, kChannel = 2 };

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also carries a
// workgroup-scope release fence, which on gfx950 waits for every outstanding global load and
// store of the wave (vmcnt(0)); the kernels here share data between waves through LDS alone,
// so global prefetches and output stores may stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier that waits only for this wave's LDS instructions: direct-to-LDS loads it
// has in flight stay in flight (the fence of lds_barrier would drain them).  Whoever consumes
// such loads waits for them (s_waitcnt vmcnt) before an earlier barrier.  The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier_keep_vm() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace gdr
