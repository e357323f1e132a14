// Vector types and small helpers shared by the MFMA kernels.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace yoco {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// the low / high bf16 of a packed pair, as float (exact: a bf16 is the top half of an fp32)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Cross-lane exchanges without LDS (gfx950 v_permlane{16,32}_swap). Called
// with the same register twice, the swap leaves lanes l and l ^ 32 (resp.
// l ^ 16) holding each other's value in one of the two results, so combining
// the pair gives the reduction over that lane pair in every lane. The whole
// wave must be active.
__device__ __forceinline__ f32x2 lane_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2 lane_pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_xor32(float x) { const f32x2 r = lane_pair32(x); return fmaxf(r[0], r[1]); }
__device__ __forceinline__ float max_xor16(float x) { const f32x2 r = lane_pair16(x); return fmaxf(r[0], r[1]); }
__device__ __forceinline__ float sum_xor32(float x) { const f32x2 r = lane_pair32(x); return r[0] + r[1]; }
__device__ __forceinline__ float sum_xor16(float x) { const f32x2 r = lane_pair16(x); return r[0] + r[1]; }

// XOR applied to the 16-byte chunk index of row r of a row-major bf16 tile that
// is read with ds_read_b64_tr_b16 (4 rows x 16 columns per 16-lane group). A
// transposing read of one wave covers 8 rows x 64 bytes; with these values its
// 16-lane groups (32 banks) and its 32-lane halves (64 banks) both hit distinct
// banks (checked exhaustively over the read pattern on the host).
// (D = 128: 0, 4, 10, 14 for r mod 4 = 0..3, as arithmetic: a table indexed at
// run time would be a memory load, which the compiler then awaits with
// everything else in flight.)
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  if constexpr (D == 128) {
    return 4 * (r & 3) + 2 * ((r >> 1) & 1);
  } else {
    return 2 * (r & 3);
  }
}

}  // namespace yoco
