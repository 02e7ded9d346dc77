// fp32 -> bf16 rounding shared by the element-wise kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

// fp32 -> bf16 bits, round to nearest even; a NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// bf16 bits -> fp32, exactly.
__device__ __forceinline__ float from_bf16(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace bi
