// nvfp4_device.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// NVFP4 element and scale formats ("Getting GLM-5.2 NVFP4 Post-Training off
// the ground", section "Going deeper: why a 4-bit weight needs two copies on
// B200"): E2M1 codes (sign in bit 3), one E4M3 scale per 16 elements, one fp32
// global scale.  The largest E2M1 magnitude (6) and E4M3 value (448) are the
// factors of the amax / (6 * 448) global scale in the
// "vroomfondel/glm-5.2-reap-504B-v2-W4A4" model card, "How it was produced".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// 16-byte streaming load that bypasses cache residency (data read once).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 bit pattern (low 16 bits of h) -> fp32, exact.
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 byte -> fp32, exact for every finite byte (subnormals included): the
// byte's exponent and mantissa fields are placed in an fp32 pattern whose
// value is 2^-120 times the E4M3 value, then rescaled by 2^120.  Bytes 0x7F /
// 0xFF (NaN) are never produced by the quantizer and are not special-cased.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    float mag = __uint_as_float((b & 0x7Fu) << 20) * 0x1p120f;
    return (b & 0x80u) ? -mag : mag;
}

// Non-negative fp32 -> E4M3 byte: round to nearest, ties to even, saturating
// at 448 (0x7E).  Below 2^-6 the E4M3 step is 2^-9, so the byte is the
// integer rint(f * 512) (which also yields 8 = 2^-6 on round-up).  Above, the
// fp32 pattern is re-biased (127 -> 7) and rounded at mantissa bit 20.
__device__ __forceinline__ uint32_t e4m3_from_f32(float f) {
    if (f < 0x1p-6f) return (uint32_t)__builtin_rintf(f * 512.0f);
    uint32_t u = __float_as_uint(f) - (120u << 23);
    uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
    return r < 0x7Eu ? r : 0x7Eu;
}

// Non-negative fp32 magnitude -> 3-bit E2M1 magnitude code, round to nearest,
// ties to the even code, saturating at 6: the number of midpoints of the grid
// {0, .5, 1, 1.5, 2, 3, 4, 6} that v passes (inclusive where the code above
// the midpoint is the even one).
__device__ __forceinline__ uint32_t e2m1_from_f32(float v) {
    return (uint32_t)(v > 0.25f) + (uint32_t)(v >= 0.75f) + (uint32_t)(v > 1.25f) +
           (uint32_t)(v >= 1.75f) + (uint32_t)(v > 2.5f) + (uint32_t)(v >= 3.5f) +
           (uint32_t)(v > 5.0f);
}

// Eight E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i)
// -> four bf16x2 pairs holding the exact grid values (no scale applied).
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t w, bf16x2 out[4]) {
    out[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    out[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    out[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    out[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
}

// Same to fp32 pairs.
__device__ __forceinline__ void fp4x8_to_f32(uint32_t w, f32x2 out[4]) {
    out[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    out[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    out[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    out[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
}

// Eight codes -> eight f16 values q * s, exact: every q * s with q an E2M1
// value and s a finite E4M3 value lies in [2^-10, 2688] with at most 6
// significant bits, which f16 represents exactly.
__device__ __forceinline__ f16x8 fp4x8_scaled_f16(uint32_t w, _Float16 s) {
    f16x2 sv = {s, s};
    f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sv;
    f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sv;
    f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sv;
    f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sv;
    return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Eight codes -> eight bf16 values q * s, exact (same argument as above; the
// fp32 product is exact and has at most 6 significant bits, so dropping the
// low 16 bits of its pattern loses nothing).
__device__ __forceinline__ uint4 fp4x8_scaled_bf16_bits(uint32_t w, float s) {
    f32x2 p[4];
    fp4x8_to_f32(w, p);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = __float_as_uint(p[i].x * s);
        uint32_t hi = __float_as_uint(p[i].y * s);
        o[i] = (lo >> 16) | (hi & 0xFFFF0000u);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Two E4M3 scale bytes (bits 0-7 and 8-15 of w) -> fp32 pair, exact, with
// the gfx950 FP8 (E4M3) -> f32 conversion.
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
}

// DPP lane shuffle of a float (lanes masked off by ROW_MASK read 0).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Maximum over each row of 16 lanes (lanes 16 q .. 16 q + 15), returned in
// every lane of the row; all lanes of the row must be active.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
    v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]: quad maxima
    v = max(v, dpp_u32<0x141>(v));   // row_half_mirror: 8-lane maxima
    v = max(v, dpp_u32<0x140>(v));   // row_mirror: 16-lane maxima
    return v;
}

// Sum over the 64 lanes of a wave with six DPP adds; the total lands in
// lane 63 (other lanes hold partial sums).
__device__ __forceinline__ float wave_sum_lane63(float v) {
    v += dpp_f32<0xB1>(v);         // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);         // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);        // row_half_mirror: 8-lane sums
    v += dpp_f32<0x140>(v);        // row_mirror: 16-lane sums
    v += dpp_f32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_f32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
        v = v > o ? v : o;
    }
    return v;
}

}  // namespace nvfp4
