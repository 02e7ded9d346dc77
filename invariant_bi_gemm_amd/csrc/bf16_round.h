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

// The RMSNorm scaling of two packed bf16 values: bf16((x * r) * g) for the
// pair in x2 with the gain pair in g2, both products rounded in fp32 (two
// separate multiplies), each result rounded to bf16 to nearest even by one
// v_cvt_pk_bf16_f32; low value in the low half.  The standalone RMSNorm and
// the GEMM that normalises its x tiles both call this, so their bf16 inputs
// to the projection are the same bits.
__device__ __forceinline__ uint32_t rms_scale_pair(uint32_t x2, float r, uint32_t g2)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    f32x2 v;
    v.x = (__uint_as_float(x2 << 16) * r) * __uint_as_float(g2 << 16);
    v.y = (__uint_as_float(x2 & 0xffff0000u) * r) * __uint_as_float(g2 & 0xffff0000u);
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint4 rms_scale_chunk(const uint4& x, float r, const uint4& g)
{
    return uint4{rms_scale_pair(x.x, r, g.x), rms_scale_pair(x.y, r, g.y), rms_scale_pair(x.z, r, g.z),
                 rms_scale_pair(x.w, r, g.w)};
}

// SwiGLU of one gate value g and its up value u: bf16(g / (1 + exp(-g)) * u),
// every step in fp32 (a correctly rounded divide, the device library's expf).
// The standalone SwiGLU kernel and the up projection that applies it in its
// epilogue both call this, so their activations are the same bits.
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u)
{
    const float sg = g / (1.0f + expf(-g));
    return to_bf16(sg * u);
}

// Four of them, packed as four bf16 in column order (low half first).
__device__ __forceinline__ uint2 swiglu4(const float* g, const float* u)
{
    uint2 p;
    p.x = (uint32_t)swiglu_bf16(g[0], u[0]) | ((uint32_t)swiglu_bf16(g[1], u[1]) << 16);
    p.y = (uint32_t)swiglu_bf16(g[2], u[2]) | ((uint32_t)swiglu_bf16(g[3], u[3]) << 16);
    return p;
}

}  // namespace bi
