// Pieces shared by the grouped-GEMM kernels (large tile, skinny, general).
#pragma once

#include "common.h"

namespace moe {

// SiLU through the hardware reciprocal (1 ulp) rather than an IEEE division:
// five instructions instead of about fifteen.  Every FFN kernel here uses this
// one definition, so a token's result does not depend on which kernel ran it.
// Both ends stay exact: exp(-z) overflowing gives -0, underflowing gives z.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Word 3 of a buffer resource on this family: 32-bit data format, raw byte addressing.
constexpr int kRsrcFlags = 0x00020000;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_ptr_t;

// A weight fragment from a tile stored k-major in LDS (rows of k, n contiguous).
// gfx950's transposing read ds_read_b64_tr_b16 works on groups of 16 lanes:
// lane i of a group receives element i % 4 of the 8-byte rows addressed by
// lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of its group, in that order (checked
// on the GPU).  With lane i of a group addressing row kb + i/4, columns
// nb + 4(i%4) .. +3, lane i receives column nb + i at rows kb .. kb+3; a second
// read four rows down gives kb+4 .. kb+7, so the lane holds eight consecutive k
// of one column: the same register contents as the fragment read from an
// n-major tile.
__device__ __forceinline__ bf16x8_t read_kn_frag(const char* p) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(p));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(p + 4 * 256));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// The same from the lane's two addresses (rows kb + i/4 and four rows down) of a
// block with its own row placement.
__device__ __forceinline__ bf16x8_t read_kn_frag2(const char* p0, const char* p1) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(p1));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace moe
