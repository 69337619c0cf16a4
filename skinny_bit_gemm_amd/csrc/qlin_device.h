// qlin_device.h -- device-side helpers shared by the quantization and GEMM
// kernels: operand vector types, the fp32 -> e4m3 / int8 code conversions,
// bf16 unpacking and rounding, and wave reductions.
//
// Quantization rules: "Building a High-Performance and Portable vLLM Linear
// Backend with Helion", section "Scope" (symmetric scales: amax over a token
// row, a 1x128 group, a channel or a 128x128 block, divided by the format's
// largest code).
#pragma once

#include <hip/hip_runtime.h>

#include "qlin_internal.h"

namespace qlin {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum { FMT_FP8 = QLIN_FP8_DYNAMIC, FMT_I8 = QLIN_W8A8_INT8, FMT_BLOCK = QLIN_BLOCK_FP8 };

// ------------------------------------------------------------ conversions

// fp32 -> fp8 E4M3FN code.  Magnitudes at or above 448 saturate to 448
// (0x7E); normal results round the 23-bit mantissa to 3 bits, nearest with
// ties to even, carrying into the exponent; below 2^-6 the value is a whole
// multiple of 2^-9, so |v| * 512 (exact) is rounded to an integer 0..8 (8 is
// the code of 2^-6).  The sign bit is copied, so -0 and tiny negatives give
// 0x80.  Inputs are finite.  All three cases are computed and one selected,
// so a wave converts without diverging.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t normal = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);   // rebias 127 -> 7
    const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    const uint32_t mag = a >= 0x43E00000u ? 0x7Eu : (a >= 0x3C800000u ? normal : sub);  // 448, 2^-6
    return sign | mag;
}

// code of one value given its row/group scale (scale 0: the run was zero,
// and so is every code; the quotient is computed anyway and discarded)
template <int FMT>
__device__ __forceinline__ uint32_t quant_code(float x, float s) {
    const float t = x / s;   // IEEE division, correctly rounded
    uint32_t code;
    if constexpr (FMT == FMT_I8) {
        float r = __builtin_rintf(t);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        code = (uint32_t)(int32_t)r & 0xFFu;
    } else {
        code = e4m3_code(t);
    }
    return s == 0.0f ? 0u : code;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, nearest with ties to even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int FMT>
__device__ __forceinline__ float qmax_of() { return FMT == FMT_I8 ? 127.0f : 448.0f; }

// Cross-lane maxima through DPP lane permutations (operand modifiers of
// ordinary vector instructions on gfx9-family targets: no LDS traffic).
// Each step takes the maximum with a permuted copy; lanes a step does not
// write keep their own value.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float max_dpp(float v) {
    const int moved = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
    return fmaxf(v, __int_as_float(moved));
}

// maximum over each row of 16 lanes, in every lane of the row:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
__device__ __forceinline__ float row16_max(float v) {
    v = max_dpp<0xB1>(v);
    v = max_dpp<0x4E>(v);
    v = max_dpp<0x141>(v);
    return max_dpp<0x140>(v);
}

// maximum over the wave (uniform): the row maxima are folded into the last
// row by row_bcast:15 (rows 1 and 3) and row_bcast:31 (rows 2 and 3), and
// read from lane 63
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    v = max_dpp<0x142, 0xA>(v);
    v = max_dpp<0x143, 0xC>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// --------------------------------------------------- activation quantization

// bf16 x 8 (one 16-byte chunk) -> max |value|.  For finite bf16 values the
// magnitude bits (sign cleared) order like the magnitudes, so the maximum is
// taken on the integer halves and converted once; the values themselves are
// not unpacked here.
__device__ __forceinline__ uint32_t absmax2_bits(uint32_t w) {
    return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}
__device__ __forceinline__ float absmax8(uint4 v) {
    const uint32_t m = max(max(absmax2_bits(v.x), absmax2_bits(v.y)),
                           max(absmax2_bits(v.z), absmax2_bits(v.w)));
    return __uint_as_float(m << 16);
}

// bf16 x 8 -> 8 codes packed little-endian into two words, one IEEE
// division per value.  The values are converted one after another: each
// division holds a scalar register pair for its scaling flag, and left to
// interleave many of them the scheduler runs out of scalar registers.
template <int FMT>
__device__ __forceinline__ uint2 quant8_ieee(uint4 v, float s) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t word = w[j >> 1];
        const float x = (j & 1) ? bf16_hi(word) : bf16_lo(word);
        out[j >> 2] |= quant_code<FMT>(x, s) << (8 * (j & 3));
        __builtin_amdgcn_sched_barrier(0);
    }
    return make_uint2(out[0], out[1]);
}

// Scales at least this large take the reciprocal route below.
constexpr float kFastScaleMin = 0x1p-60f;

// a / s for a >= 0, from y = 1 / s (an IEEE division, correctly rounded):
// q0 = a*y is within 1.5 ulp of a/s, one residual correction makes it
// faithful, and a second one (Markstein's theorem: a faithful quotient, a
// reciprocal within 2^-24 relative error, exact FMA residual) rounds it
// correctly, so the result is the IEEE quotient a / s.  Only when a is so
// small (below about 2^-102) that the residuals lose bits to underflow may
// the last bit differ; with s >= 2^-60 the quotient is then below 2^-42,
// far from the first rounding threshold of either code, so the code is the
// same.  (Checked on gfx950 over every bf16 amax and every bf16 x <= amax,
// for both 127 and 448: identical int8 and e4m3 codes.)
__device__ __forceinline__ float div_by_scale(float a, float s, float y) {
    const float q0 = a * y;
    const float r0 = __builtin_fmaf(-s, q0, a);
    const float q1 = __builtin_fmaf(r0, y, q0);
    const float r1 = __builtin_fmaf(-s, q1, a);
    return __builtin_fmaf(r1, y, q1);
}

// bf16 x 8 -> 8 codes packed little-endian into two words, given the run's
// scale s and y = 1.0f / s.  The quotient is formed for |x| and the sign of
// x copied onto it (the division, the rounding and the saturation are all
// symmetric, and -0 keeps its sign as code 0x80); e4m3 codes come from the
// matrix core's conversion instruction (round to nearest even, subnormals
// kept; identical to e4m3_code for every fp32 of magnitude <= 448, which the
// clamp guarantees).
template <int FMT>
__device__ __forceinline__ uint2 quant8(uint4 v, float s, float y) {
    if (!(s >= kFastScaleMin)) return quant8_ieee<FMT>(v, s);   // tiny or zero scale
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t word = w[2 * h + (j >> 1)];
            const uint32_t bits = (j & 1) ? (word & 0xFFFF0000u) : (word << 16);
            float q = div_by_scale(__uint_as_float(bits & 0x7FFFFFFFu), s, y);
            if constexpr (FMT == FMT_I8) q = __builtin_rintf(fminf(q, 127.0f));
            else q = fminf(q, 448.0f);
            t[j] = __uint_as_float(__float_as_uint(q) | (bits & 0x80000000u));
        }
        if constexpr (FMT == FMT_I8) {
            out[h] = ((uint32_t)(int32_t)t[0] & 0xFFu) | (((uint32_t)(int32_t)t[1] & 0xFFu) << 8) |
                     (((uint32_t)(int32_t)t[2] & 0xFFu) << 16) | ((uint32_t)(int32_t)t[3] << 24);
        } else {
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], pk, true);
            out[h] = (uint32_t)pk;
        }
    }
    return make_uint2(out[0], out[1]);
}

// y = 1 / s for quant8 (any value for a scale that takes the IEEE route)
__device__ __forceinline__ float recip_scale(float s) {
    return s >= kFastScaleMin ? 1.0f / s : 0.0f;
}

}  // namespace qlin
