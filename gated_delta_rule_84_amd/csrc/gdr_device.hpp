// gdr_device.hpp -- small device helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Element `i` of an array that is bf16 (is_bf16 != 0) or fp32.
__device__ __forceinline__ float ld_elem(const void *p, long i, int is_bf16) {
    return is_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(p)[i])
                   : static_cast<const float *>(p)[i];
}

__device__ __forceinline__ void st_elem(void *p, long i, float x, int is_bf16) {
    if (is_bf16)
        static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
    else
        static_cast<float *>(p)[i] = x;
}

}  // namespace gdr
