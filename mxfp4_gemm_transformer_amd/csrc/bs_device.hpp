// Device-side building blocks for the gfx950 kernels: vector types, the
// e4m3fn encoder, bf16 rounding, the tanh-GELU epilogue, and the operand
// layout of the scaled MFMA instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum { EPI_NONE = 0, EPI_BIAS = 1, EPI_BIAS_GELU_TANH = 2 };

// Operand formats of V_MFMA_SCALE_F32_*_F8F6F4 (cbsz / blgp encodings).
enum { MFMA_FMT_FP8 = 0, MFMA_FMT_FP4 = 4 };

// E8M0 byte that scales by 1.0.
constexpr int E8M0_ONE = 127;

// ---------------------------------------------------------------- e4m3fn
// Nearest e4m3fn code to a finite fp32 value, ties to the even mantissa,
// saturating at +-448 (0x7E / 0xFE), sign kept (also for zero results).
// Normal range: round the binary32 pattern to 3 mantissa bits by adding
// 0x7FFFF plus the kept LSB (carry propagates into the exponent), then
// rebias the exponent from 127 to 7. Below 2^-6 the e4m3 grid is uniform
// with step 2^-9, so the code is rint(|v| * 2^9) (exact scaling, the
// hardware rint rounds to nearest even).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    const uint32_t bits = __float_as_uint(v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t mag = bits & 0x7FFFFFFFu;
    uint32_t code;
    if (mag >= 0x43E00000u) {                 // |v| >= 448
        code = 0x7Eu;
    } else if (mag < 0x3C800000u) {           // |v| < 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
    } else {
        const uint32_t r = mag + 0x7FFFFu + ((mag >> 20) & 1u);
        code = (r >> 20) - (120u << 3);       // (127 - 7) << 3
    }
    return sign | code;
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even, by gfx950's V_CVT_PK_BF16_F32.
// Measured on MI355X over every finite fp32 bit pattern (x and -x as a
// pair): identical to rounding the binary32 pattern by adding 0x7FFF plus
// the kept LSB and dropping the low 16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two values in one conversion: lo in bits 0-15, hi in bits 16-31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const v2f v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, v2bf));
}

// -------------------------------------------------------------- epilogue
// 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3). With
// tanh(u) = 1 - 2 / (e^(2u) + 1), 1 + tanh(u) = 2 - 2 / (e^(2u) + 1), so
// GELU = v - v / (e^(2u) + 1): one hardware exp2 and one reciprocal. The
// exponent is clamped so e^(2u) stays finite; past |u| = 15 tanh is +-1 to
// fp32 precision. Relative error is a few fp32 ulps, far below the bf16
// rounding of the output.
__device__ __forceinline__ float gelu_tanh(float v) {
    const float u = 0.7978845608028654f * (v + 0.044715f * v * v * v);
    const float t = fminf(fmaxf(2.0f * 1.4426950408889634f * u, -43.28f), 43.28f);  // 2u log2(e)
    const float e = __builtin_amdgcn_exp2f(t);
    return v - v * __builtin_amdgcn_rcpf(e + 1.0f);
}

// The epilogue after the per-token scale: + bias, then GELU.
__device__ __forceinline__ float epilogue_rest(float v, float bias, int epi) {
    if (epi != EPI_NONE) v += bias;
    if (epi == EPI_BIAS_GELU_TANH) v = gelu_tanh(v);
    return v;
}

__device__ __forceinline__ float epilogue(float acc, float a_scale, float bias, int epi) {
    return epilogue_rest(a_scale * acc, bias, epi);
}

// With a per-output-channel weight scale cs (1 when the weights carry E8M0
// block scales instead: the product is then exact).
__device__ __forceinline__ float epilogue(float acc, float a_scale, float cs, float bias, int epi) {
    return epilogue_rest(a_scale * acc * cs, bias, epi);
}

// ------------------------------------------------------ MFMA operand layout
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 (measured on gfx950):
//   lane l = i + 16 g (i = row of A / column of B, g = 0..3).
//   fp8 operand, K window [k0, k0 + 128):
//     VGPRs 0-3 hold k0 + 16 g + [0, 16), VGPRs 4-7 hold k0 + 64 + 16 g + [0, 16)
//   fp4 operand: VGPRs 0-3 hold the 32 elements k0 + 32 g + [0, 32), two per
//     byte, low nibble first (the packed row-major layout, unchanged)
//   E8M0 scale of lane l applies to the 32-element block k0 + 32 g + [0, 32)
//     of row/column i.
//   D: lane l, VGPR v -> row 4 g + v, column i.
// V_MFMA_SCALE_F32_32X32X64_F8F6F4: lane l = i + 32 g (g = 0..1), window of
//   64: fp8 VGPRs 0-3 hold k0 + 16 g + [0,16), VGPRs 4-7 hold k0 + 32 + 16 g
//   + [0, 16); fp4 holds k0 + 32 g + [0, 32); the scale of lane l covers
//   block k0 + 32 g + [0, 32); D: lane l, VGPR v -> row 8 (v / 4) + 4 g +
//   v % 4, column i.
template <bool FP4>
__device__ __forceinline__ v4f mfma16(const v8i &a, const v8i &b, const v4f &c, int sa, int sb) {
    if (FP4)
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, MFMA_FMT_FP8, MFMA_FMT_FP4,
                                                                0, sa, 0, sb);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, MFMA_FMT_FP8, MFMA_FMT_FP8, 0,
                                                            sa, 0, sb);
}

template <bool FP4>
__device__ __forceinline__ v16f mfma32(const v8i &a, const v8i &b, const v16f &c, int sa, int sb) {
    if (FP4)
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, MFMA_FMT_FP8, MFMA_FMT_FP4, 0,
                                                               sa, 0, sb);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, MFMA_FMT_FP8, MFMA_FMT_FP8, 0,
                                                           sa, 0, sb);
}

// The same instruction with the weights as the A operand (their format and
// E8M0 scale on the A side) and e4m3 activations as B with unit scales; the
// result is the transposed tile: D row = weight row, D column = token.
template <bool FP4>
__device__ __forceinline__ v16f mfma32_wt(const v8i &w, const v8i &a, const v16f &c, int sw) {
    if (FP4)
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, c, MFMA_FMT_FP4, MFMA_FMT_FP8, 0,
                                                               sw, 0, E8M0_ONE);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, c, MFMA_FMT_FP8, MFMA_FMT_FP8, 0,
                                                           sw, 0, E8M0_ONE);
}

// Both operands' formats chosen (W4A4: fp4 activations with their own
// per-lane E8M0 scales).
template <bool FP4W, bool FP4A>
__device__ __forceinline__ v4f mfma16x(const v8i &a, const v8i &b, const v4f &c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        a, b, c, FP4A ? MFMA_FMT_FP4 : MFMA_FMT_FP8, FP4W ? MFMA_FMT_FP4 : MFMA_FMT_FP8, 0, sa, 0, sb);
}

// Weights as the instruction's A operand (scale sw), activations as its B
// operand (scale sa: E8M0_ONE for e4m3 activations). SEL picks the byte of
// each 32-bit scale operand the instruction uses (measured on gfx950: byte
// SEL, little-endian).
template <bool FP4W, bool FP4A, int SEL = 0>
__device__ __forceinline__ v16f mfma32_wt2(const v8i &w, const v8i &a, const v16f &c, int sw, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        w, a, c, FP4W ? MFMA_FMT_FP4 : MFMA_FMT_FP8, FP4A ? MFMA_FMT_FP4 : MFMA_FMT_FP8, SEL, sw,
        FP4A ? SEL : 0, sa);
}

__device__ __forceinline__ v8i pack8(const uint4 &lo, const uint4 &hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

__device__ __forceinline__ uint4 ldg16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

}  // namespace bsg
