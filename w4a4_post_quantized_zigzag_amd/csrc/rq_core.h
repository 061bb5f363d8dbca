// Arithmetic of the per-step rotate-quantize shared by the streaming rotate-quantize kernel and by
// the GEMM epilogue that quantizes the next linear's input: the block rotation x'^T = R_b^T x^T on
// v_mfma_f32_16x16x32_f16 with the two-part R (R ~= hi + lo 2^-12), the step scale lookup, and the
// fp32 quantization with int4 packing. Both callers use these functions with the same fragment
// order, so for the same fp16 inputs they produce the same codes bit for bit.
//
// Rotation before quantization: gist.science summary, "Metodologia" item 1 (R_b = U_b H_B);
// the per-step scale lookup: vnrobo.com "Y tuong paper".
#pragma once

#include "w4a4_internal.h"

namespace w4a4 {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// A per-step table entry and its reciprocal fp32(1/s). Only a positive finite entry is a scale.
// Any other entry (zero, negative, infinite or NaN: an uncalibrated or damaged table) yields the
// scale NaN and the reciprocal 0, so every code becomes 0 and every output of the GEMM that
// consumes them is NaN: the failure shows in the result instead of a plausible-looking value.
struct StepScale {
    float s, rcp;
};
__device__ __forceinline__ StepScale step_scale(const float *table, int idx)
{
    const float s = table[idx];
    if (s > 0.0f && s <= 3.402823466e38f) return StepScale{s, (float)(1.0 / (double)s)};
    return StepScale{__builtin_nanf(""), 0.0f};
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

// R_b^T fragments of the output channels jbase + 16 jf .. + 15 of block b (KK = B / 32 k steps of
// 32 inputs). The high part is scaled by 2^12 (exact, as |R| <= 1), so that x.hi and x.lo
// accumulate in one fp32 accumulator at the same scale.
template <int JF, int KK>
__device__ __forceinline__ void load_rot_frags(const _Float16 *__restrict__ rhi,
                                               const _Float16 *__restrict__ rlo, int b, int jbase,
                                               int lane, int B, v8h (&ahi)[JF][KK],
                                               v8h (&alo)[JF][KK])
{
#pragma unroll
    for (int jf = 0; jf < JF; ++jf)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int64_t off = rot16_fragment(b, jbase / 16 + jf, kk, lane, B);
            ahi[jf][kk] = *reinterpret_cast<const v8h *>(rhi + off) * (_Float16)(1 << ROT_LO_SHIFT);
            alo[jf][kk] = *reinterpret_cast<const v8h *>(rlo + off);
        }
}

// acc[mf][jf] = 2^12 x' for tokens mf*16 + (lane % 16) and channels jbase + 16 jf + 4 (lane / 16)
// + 0..3, from the input fragments load_x(mf, kk) (the 8 inputs 8 (4 kk + lane / 16) .. + 7 of
// token mf*16 + lane % 16). For each k step the low-part products of every accumulator come first,
// then the high-part ones. Each of those two groups is MF * JF independent MFMAs, kept together
// by scheduling barriers (left alone, the compiler regroups them into per-accumulator chains of
// dependent MFMAs and runs at the matrix pipe's latency); the next step's inputs are read ahead.
template <int MF, int JF, int KK, typename LoadX>
__device__ __forceinline__ void rotate_acc(const v8h (&ahi)[JF][KK], const v8h (&alo)[JF][KK],
                                           LoadX &&load_x, v4f (&acc)[MF][JF])
{
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int jf = 0; jf < JF; ++jf) acc[mf][jf] = v4f{0.f, 0.f, 0.f, 0.f};
    v8h xb[2][MF];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) xb[0][mf] = load_x(mf, 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const int c = kk & 1;
        if (kk + 1 < KK) {
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) xb[c ^ 1][mf] = load_x(mf, kk + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
            for (int jf = 0; jf < JF; ++jf)
                acc[mf][jf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[jf][kk], xb[c][mf], acc[mf][jf], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
            for (int jf = 0; jf < JF; ++jf)
                acc[mf][jf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[jf][kk], xb[c][mf], acc[mf][jf], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace w4a4
