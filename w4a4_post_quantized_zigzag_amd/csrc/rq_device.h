// Device helpers shared by the rotate-quantize kernels and the GEMM epilogue that rotates and
// quantizes a tile for the next linear: the step scale lookup, the fp32 quantize-and-pack of four
// rotated values, and the vector types of the fp16 MFMA operands.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace w4a4 {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float step_scale(const float *table, int step)
{
    float s = table[step];
    return (s > 0.0f && s <= 3.402823466e38f) ? s : 1.0f;
}

// Four rotated values held as acc = 2^12 x' -> four int4 codes packed low nibble first in the low
// 16 bits (the bits above are garbage). rs = 2^-12 * fp32(1/s), so acc * rs is the fp32 product
// x' * fp32(1/s) rounded once (both power-of-two scalings are exact for any x' and 1/s that can
// give a nonzero code). Adding 1.5 * 2^23 rounds that product to an integer, ties to even, and
// leaves the integer in the low mantissa bits; the clamp to [-8, 7] is applied in that form and
// the two's-complement nibble is read off the bit pattern.
// Q8: int8 codes, clamp to [-128, 127] and one byte per code (four bytes returned).
template <bool Q8 = false>
__device__ __forceinline__ uint32_t quant_pack4(v4f acc, float rs)
{
#pragma clang fp contract(off)
    constexpr float MAGIC = 12582912.0f;
    constexpr float LOQ = Q8 ? -128.0f : -8.0f, HIQ = Q8 ? 127.0f : 7.0f;
    uint32_t n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float y = acc[i] * rs;
        float f = y + MAGIC;
        f = fminf(fmaxf(f, MAGIC + LOQ), MAGIC + HIQ);
        n[i] = __float_as_uint(f);
    }
    if (Q8)
        return (n[0] & 0xFFu) | ((n[1] & 0xFFu) << 8) | ((n[2] & 0xFFu) << 16) | (n[3] << 24);
    uint32_t t = (n[0] & 0xFu) | ((n[1] << 4) & ~0xFu);
    t = (t & 0xFFu) | ((n[2] << 8) & ~0xFFu);
    return (t & 0xFFFu) | ((n[3] << 12) & ~0xFFFu);
}

}  // namespace w4a4
