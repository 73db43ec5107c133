// gdr_mfma.hpp -- matrix-core and LDS-copy primitives shared by the gfx950 kernels.
//
// v_mfma_f32_16x16x32_bf16 lane layout (lane = 16 q + r, q in 0..3, r in 0..15):
//   A (16 x 32): lane holds A[r][8q .. 8q+7];  B (32 x 16): B[8q .. 8q+7][r];
//   C (16 x 16): lane holds C[4q .. 4q+3][r].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void *lds_void_t;
typedef __attribute__((address_space(1))) void *gbl_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 *lds_i16x4_t;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// two fp32 -> two bf16 (round to nearest even) in one packed conversion
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// 16 bytes per lane, global -> LDS; lane l writes dst + 16 l (dst wave-uniform).
// Completion is counted by vmcnt like any vector load.
__device__ __forceinline__ void dma16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)dst, 16, 0, 0);
}

}  // namespace gdr
