// nvfp4_encode.hpp -- the NVFP4 block encoder shared by the quantize kernels
// and the GEMV that quantizes its activation in registers.
//
// Scale rule and element rounding: "vroomfondel/glm-5.2-reap-504B-v2-W4A4"
// model card, "How it was produced", and "Getting GLM-5.2 NVFP4
// Post-Training off the ground", "Going deeper".  Given Sg and t = 6 Sg:
// s_f = bmax / t, s8 = E4M3(s_f), d = s * Sg, code = sign | E2M1(|x| / d),
// each fp32 step rounded on its own (no contraction inside these functions).
#pragma once

#include "nvfp4_device.hpp"

namespace nvfp4 {

// Magnitude code of one bf16 element under divisor d (d == 0 -> 0), sign in
// bit 3, with IEEE division.  Used for blocks whose divisor lies outside the
// range of the exact reciprocal path below.
__device__ __forceinline__ uint32_t encode_elem(uint32_t h, float d) {
#pragma clang fp contract(off)
    float v = (d > 0.0f) ? bf16_to_f32(h & 0x7FFFu) / d : 0.0f;
    return ((h >> 12) & 8u) | e2m1_from_f32(v);
}

// The fp32 quotient a / d for the E2M1 rounding decision, without a divide
// instruction, for bf16 a with |a| <= 8 d, d in [2^-100, 2^125) and
// y = RN(1 / d): q0 = a * y is within a few ulps, the fma gives the remainder
// q0 * d - a exactly, and one Newton-Markstein correction
// q0 - (q0 * d - a) * y is faithful (within one ulp of a / d, same sign).  A
// one-ulp difference from RN(a / d) can change the E2M1 code only next to a
// midpoint of the E2M1 grid, and there the corrected quotient equals
// RN(a / d): the codes are those of the IEEE quotient (checked on the host
// for every bf16 numerator).  The bounds keep y, the quotient and the
// remainder clear of overflow and of the subnormal range where the remainder
// stops being exact; the remainder is formed as q0 * d - a so that a zero a
// keeps its sign.
__device__ __forceinline__ float div_e2m1(float a, float d, float y) {
#pragma clang fp contract(off)
    const float q0 = a * y;
    const float n0 = __builtin_fmaf(q0, d, -a);
    return __builtin_fmaf(-n0, y, q0);
}

// Two bf16 elements (one 32-bit word) -> their E2M1 codes in byte SEL of acc.
// The gfx950 fp32 -> fp4 conversion (scale 1) rounds to nearest even on the
// E2M1 grid, saturates at 6 and keeps the sign, also on a zero result, so
// converting the signed quotient x / d gives sign | E2M1(|x| / d).
template <int SEL>
__device__ __forceinline__ uint32_t encode_pair(uint32_t acc, uint32_t w, float d, float y) {
#pragma clang fp contract(off)
    const float ql = div_e2m1(__uint_as_float(w << 16), d, y);
    const float qh = div_e2m1(__uint_as_float(w & 0xFFFF0000u), d, y);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, ql, qh, 1.0f, SEL);
}

// The per-block half of the encoder, for kernels that hold one element of a
// block per lane: the scale byte, its value s, the divisor d = s * Sg and
// whether the reciprocal quotient applies (the block-level condition of
// encode_block below), given the block's magnitude maximum as a bf16 pattern.
struct BlockEnc {
    uint32_t s8;
    float s, d, y;
    bool fast;
};

__device__ __forceinline__ BlockEnc block_enc(uint32_t max_bits, float Sg, float t) {
#pragma clang fp contract(off)
    const float bmax = bf16_to_f32(max_bits);
    const float s_f = (t > 0.0f) ? bmax / t : 0.0f;
    BlockEnc b;
    b.s8 = e4m3_from_f32(s_f);
    b.s = e4m3_to_f32(b.s8);
    b.d = b.s * Sg;
    b.fast = b.d >= 0x1p-100f && b.d < 0x1p125f && bmax <= 8.0f * b.d;
    b.y = b.fast ? 1.0f / b.d : 0.0f;
    return b;
}

// The 4-bit code (sign in bit 3) of one bf16 element h of a block, with the
// same quotient and rounding as encode_block.
__device__ __forceinline__ uint32_t encode_one(uint32_t h, const BlockEnc& b) {
#pragma clang fp contract(off)
    if (b.d == 0.0f) return (h >> 12) & 0x8u;   // magnitude 0, the sign remains
    if (b.fast) {
        const float q = div_e2m1(bf16_to_f32(h & 0xFFFFu), b.d, b.y);
        return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q, 0.0f, 1.0f, 0) & 0xFu;
    }
    return encode_elem(h & 0xFFFFu, b.d);
}

// One 16-element block: 8 words of bf16 pairs -> 8 code bytes + scale byte.
__device__ __forceinline__ uint32_t encode_block(const uint32_t w[8], float Sg, float t, uint2& out) {
#pragma clang fp contract(off)
    u16x2 m = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
    const float bmax = bf16_to_f32(m.x > m.y ? m.x : m.y);
    const float s_f = (t > 0.0f) ? bmax / t : 0.0f;
    const uint32_t s8 = e4m3_from_f32(s_f);
    const float d = e4m3_to_f32(s8) * Sg;
    if (d == 0.0f) {
        // zero divisor (an all-zero block, a zero global scale, or a scale
        // that rounds to 0): every magnitude code is 0, only the signs remain
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j >> 2] |= (((w[j] >> 12) & 0x08u) | ((w[j] >> 24) & 0x80u)) << (8 * (j & 3));
        out = make_uint2(o[0], o[1]);
        return s8;
    }
    // Fast path when the quotient conditions hold for every element
    // (|x| <= bmax <= 8 d): all blocks of ordinary tensors.  Saturated scales,
    // zero blocks and extreme global scales take the IEEE division.
    if (d >= 0x1p-100f && d < 0x1p125f && bmax <= 8.0f * d) {
        const float y = 1.0f / d;
        uint32_t o0 = 0u, o1 = 0u;
        o0 = encode_pair<0>(o0, w[0], d, y);
        o0 = encode_pair<1>(o0, w[1], d, y);
        o0 = encode_pair<2>(o0, w[2], d, y);
        o0 = encode_pair<3>(o0, w[3], d, y);
        o1 = encode_pair<0>(o1, w[4], d, y);
        o1 = encode_pair<1>(o1, w[5], d, y);
        o1 = encode_pair<2>(o1, w[6], d, y);
        o1 = encode_pair<3>(o1, w[7], d, y);
        out = make_uint2(o0, o1);
    } else {
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t byte = encode_elem(w[j] & 0xFFFFu, d) | (encode_elem(w[j] >> 16, d) << 4);
            o[j >> 2] |= byte << (8 * (j & 3));
        }
        out = make_uint2(o[0], o[1]);
    }
    return s8;
}

}  // namespace nvfp4
