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

// XOR applied to the 16-byte chunk index of row r of a row-major bf16 tile that
// is read with ds_read_b64_tr_b16 (4 rows x 16 columns per 16-lane group). A
// transposing read of one wave covers 8 rows x 64 bytes; with these values its
// 16-lane groups (32 banks) and its 32-lane halves (64 banks) both hit distinct
// banks (checked exhaustively over the read pattern on the host).
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  if constexpr (D == 128) {
    constexpr int t[4] = {0, 4, 10, 14};
    return t[r & 3];
  } else {
    return 2 * (r & 3);
  }
}

}  // namespace yoco
