// Internal helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 storage: the high half of an IEEE float32

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// 16 bytes as a native vector: selects and copies of it stay in registers
// (HIP's uint4 is a struct, which a conditional expression can push to scratch)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// float32 -> bfloat16, round to nearest, ties to even, by the hardware
// conversion (v_cvt_pk_bf16_f32); a NaN stays a NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// two floats -> two bfloat16 in one word (a in the low half), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kPerVec = 8;  // elements in 16 bytes
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f32(float f) { return f32_to_bf16(f); }
};
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float f) { return f; }
};

// Unpack 16 bytes of T into float32 lanes.
__device__ __forceinline__ void unpack16(const uint4& v, bf16_t, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4& v, float, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ uint4 pack16(const float* f, bf16_t) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = uint32_t(f32_to_bf16(f[2 * i])) | (uint32_t(f32_to_bf16(f[2 * i + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint4 pack16(const float* f, float) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Block barrier without the memory drain of __syncthreads(): waves meet, but
// loads in flight stay in flight (callers wait on their own counters first).
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Lanes below this one.
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << lane_id()) - 1;
}

// Lanes of the wave whose `key` equals this lane's (key in [0, 2^bits)).
__device__ __forceinline__ uint64_t match_any(uint32_t key, int bits, uint64_t active) {
  uint64_t m = active;
  for (int b = 0; b < bits; ++b) {
    const uint64_t set = __ballot((key >> b) & 1u);
    m &= ((key >> b) & 1u) ? set : ~set;
  }
  return m;
}

}  // namespace moe
