/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for NVFP4 quantization and the
 * block-scaled products that consume it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source, header, table or constant generator
 * with the HIP library; it is written from the format definitions on the
 * pages, step by step, with no blocking, fusion or reordering.
 *
 * Sources (page title -> section):
 *  [P1] "Getting GLM-5.2 NVFP4 Post-Training off the ground"
 *       -> "Going deeper: why a 4-bit weight needs two copies on B200":
 *          NVFP4 = E2M1 4-bit values + one FP8 E4M3 scale per 16-element
 *          block along the contraction axis + one FP32 global scale; codes
 *          bit-packed two per byte; Fprop Y = X * W^T with K innermost.
 *       -> "The bottom line": block scales come from the block maximum.
 *  [P2] "GLM-5.2-NVFP4" model card -> "Quantization recipe": block size 16,
 *       FP4 weights + FP8 block scales.
 *  [P3] "vroomfondel/glm-5.2-reap-504B-v2-W4A4" model card
 *       -> "How it was produced": e2m1 fp4, per-16 e4m3 block scales, linear
 *          block-scale layout, per-tensor fp32 global scale equal to the
 *          tensor amax over (6 * 448); a static per-tensor input_scale for the
 *          activations of the W4A4 path.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *  - E2M1 = sign, 2 exponent bits (bias 1), 1 mantissa bit: magnitudes
 *    {0, .5, 1, 1.5, 2, 3, 4, 6}; E4M3 is the "fn" variant (max 448, no inf).
 *    Both maxima are fixed by the 6*448 divisor of the global scale.
 *  - Rounding is round-to-nearest, ties to the even code, saturating at the
 *    format maximum (no stochastic rounding).
 *  - fp32 step order: Sg = amax / 2688; t = 6 * Sg; per block s_f = bmax / t,
 *    s8 = E4M3(s_f), s = decode(s8); per element d = s * Sg, v = x / d,
 *    code = sign(x) | E2M1(|v|).  A zero divisor gives magnitude code 0.
 *  - Even element in the low nibble; scales stored [rows, cols/16] row-major.
 *  - Products are accumulated in fp64 over the dequantized operands (an exact
 *    reference for kernels that accumulate in fp32).
 *
 * Floating-point discipline: build with -O2 -fno-fast-math -ffp-contract=off
 * so every float operation below is one IEEE-754 binary32 operation with
 * round-to-nearest-even and no fused multiply-add.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ---------------------------------------------------------------------- */
/* Element formats                                                         */
/* ---------------------------------------------------------------------- */

/* E2M1 magnitudes indexed by the 3 low bits of a code. [P1] "Going deeper". */
static const double ORC_E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Value of a 4-bit E2M1 code: bit 3 is the sign. */
ORC_API double orc_e2m1_value(uint32_t code) {
    double m = ORC_E2M1_MAG[code & 7u];
    return (code & 8u) ? -m : m;
}

/* Value of an E4M3 ("fn") byte: sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN.  The largest
 * finite value is 0x7E = 448, the divisor's second factor in [P3]. */
ORC_API double orc_e4m3_value(uint32_t b) {
    uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
    double v;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -v : v;
}

/* E4M3 encode of a non-negative float: the nearest finite E4M3 value, ties
 * to the even byte (= even mantissa), saturating at 448.  Written as a search
 * over all 127 non-negative finite values.  Distances are taken in double;
 * for the inputs that can sit near a grid value they are exact, so ties are
 * detected exactly. */
ORC_API uint32_t orc_e4m3_encode(float f) {
    if (!(f >= 0.0f)) return 0u;            /* precondition: f >= 0 (NaN -> 0) */
    if (f > 448.0f) return 0x7Eu;           /* saturate (also catches +inf) */
    uint32_t best = 0u;
    double bestd = (double)f;               /* distance to 0.0 (byte 0) */
    for (uint32_t b = 1u; b <= 0x7Eu; b++) {
        double d = fabs((double)f - orc_e4m3_value(b));
        if (d < bestd || (d == bestd && (b & 1u) == 0u)) {
            best = b;
            bestd = d;
        }
    }
    return best;
}

/* E2M1 encode of a non-negative float magnitude: nearest of the 8
 * magnitudes, ties to the even code, saturating at 6 (code 7). */
ORC_API uint32_t orc_e2m1_encode_mag(float v) {
    if (!(v >= 0.0f)) return 0u;
    if (v > 6.0f) return 7u;
    uint32_t best = 0u;
    double bestd = (double)v;
    for (uint32_t c = 1u; c < 8u; c++) {
        double d = fabs((double)v - ORC_E2M1_MAG[c]);
        if (d < bestd || (d == bestd && (c & 1u) == 0u)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* Batch forms used by the brute-force pins. */
ORC_API void orc_e4m3_encode_array(const float* f, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)orc_e4m3_encode(f[i]);
}
ORC_API void orc_e2m1_encode_mag_array(const float* f, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)orc_e2m1_encode_mag(f[i]);
}

/* bf16 <-> fp32.  bf16 is the top half of an fp32 bit pattern. */
ORC_API float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite float to the nearest bf16, ties to even: compare the two
 * bf16 neighbours of f (truncation and the next magnitude up). */
ORC_API uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t lo = (uint16_t)(u >> 16);                 /* toward zero */
    uint16_t hi = (uint16_t)(lo + 1u);                 /* next magnitude */
    double dlo = fabs((double)f - (double)orc_bf16_to_f32(lo));
    double dhi = fabs((double)f - (double)orc_bf16_to_f32(hi));
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1u) ? hi : lo;
}

ORC_API void orc_f32_to_bf16_array(const float* f, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16(f[i]);
}

/* Round a finite double to the nearest bf16, ties to even (no intermediate
 * rounding to fp32): the answer is one of the three bf16 values around the
 * truncation of (float)v, compared by exact double distance. */
ORC_API uint16_t orc_f64_to_bf16(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t c = (uint16_t)(u >> 16);
    uint16_t cand[3] = {(uint16_t)(c - 1u), c, (uint16_t)(c + 1u)};
    uint16_t best = c;
    double bestd = fabs(v - (double)orc_bf16_to_f32(c));
    for (int i = 0; i < 3; i++) {
        if ((cand[i] & 0x7FFFu) > 0x7F7Fu) continue;   /* skip inf / NaN patterns */
        if ((cand[i] & 0x8000u) != (c & 0x8000u)) continue;
        double d = fabs(v - (double)orc_bf16_to_f32(cand[i]));
        if (d < bestd || (d == bestd && (cand[i] & 1u) == 0u)) {
            best = cand[i];
            bestd = d;
        }
    }
    return best;
}

/* ---------------------------------------------------------------------- */
/* Quantize / dequantize  ([P3] "How it was produced"; [P1] "Going deeper") */
/* ---------------------------------------------------------------------- */

/* Per-tensor global scale of the dynamic mode: fl(amax / (6 * 448)). */
ORC_API float orc_global_scale(const uint16_t* x, int64_t n) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(orc_bf16_to_f32(x[i]));
        if (a > amax) amax = a;
    }
    return amax / 2688.0f;
}

/* Quantize a row-major bf16 [rows, cols] tensor (cols % 16 == 0) under the
 * given global scale Sg.  codes: [rows, cols/2] (even element in the low
 * nibble); scales: [rows, cols/16] E4M3 bytes. */
ORC_API void orc_quantize(const uint16_t* x, int64_t rows, int64_t cols, float Sg,
                          uint8_t* codes, uint8_t* scales) {
    const float t = 6.0f * Sg;
    const int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const uint16_t* xb = x + r * cols + b * 16;
            float bmax = 0.0f;
            for (int k = 0; k < 16; k++) {
                float a = fabsf(orc_bf16_to_f32(xb[k]));
                if (a > bmax) bmax = a;
            }
            float s_f = (t > 0.0f) ? bmax / t : 0.0f;
            uint32_t s8 = orc_e4m3_encode(s_f);
            float s = (float)orc_e4m3_value(s8);
            float d = s * Sg;
            uint8_t nib[16];
            for (int k = 0; k < 16; k++) {
                float xv = orc_bf16_to_f32(xb[k]);
                float v = (d > 0.0f) ? fabsf(xv) / d : 0.0f;
                nib[k] = (uint8_t)((signbit(xv) ? 8u : 0u) | orc_e2m1_encode_mag(v));
            }
            for (int j = 0; j < 8; j++)
                codes[r * (cols / 2) + b * 8 + j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
            scales[r * nb + b] = (uint8_t)s8;
        }
    }
}

/* Dequantized element as fp32: fl(fl(q * s) * Sg).  q * s is exact. */
static float orc_deq_elem(const uint8_t* codes, const uint8_t* scales, float Sg,
                          int64_t cols, int64_t r, int64_t k) {
    uint8_t byte = codes[r * (cols / 2) + k / 2];
    uint32_t code = (k & 1) ? (uint32_t)(byte >> 4) : (uint32_t)(byte & 15u);
    float q = (float)orc_e2m1_value(code);
    float s = (float)orc_e4m3_value(scales[r * (cols / 16) + k / 16]);
    float qs = q * s;
    return qs * Sg;
}

/* Dequantize to fp32 [rows, cols]; optionally also to bf16 (RNE). */
ORC_API void orc_dequantize(const uint8_t* codes, const uint8_t* scales, float Sg,
                            int64_t rows, int64_t cols, float* out_f32, uint16_t* out_bf16) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < cols; k++) {
            float v = orc_deq_elem(codes, scales, Sg, cols, r, k);
            if (out_f32) out_f32[r * cols + k] = v;
            if (out_bf16) out_bf16[r * cols + k] = orc_f32_to_bf16(v);
        }
}

/* ---------------------------------------------------------------------- */
/* Products ([P1] "Going deeper" / "TN, NT": Y = X * W^T, K innermost)      */
/* ---------------------------------------------------------------------- */

/* W4A16: y[m, n] = sum_k deq(W)[n, k] * x[m, k], fp64 accumulation.
 * x: bf16 [M, K]; W: NVFP4 [N, K]; y: double [M, N]. */
ORC_API void orc_gemv_w4a16(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                            const uint8_t* w_codes, const uint8_t* w_scales, float w_global,
                            double* y) {
    float* wd = (float*)malloc(sizeof(float) * (size_t)N * (size_t)K);
    float* xf = (float*)malloc(sizeof(float) * (size_t)M * (size_t)K);
    orc_dequantize(w_codes, w_scales, w_global, N, K, wd, NULL);
    for (int64_t i = 0; i < M * K; i++) xf[i] = orc_bf16_to_f32(x[i]);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) acc += (double)wd[n * K + k] * (double)xf[m * K + k];
            y[m * N + n] = acc;
        }
    free(wd);
    free(xf);
}

/* W4A4: X is quantized under the static per-tensor input_scale, both
 * operands are dequantized, and y = X^ * W^^T in fp64.  [P3] "How it was
 * produced" (static input_scale) and "Kernel choice" (W4A4 path). */
ORC_API void orc_gemm_w4a4(const uint16_t* x, float input_scale, int64_t M, int64_t N, int64_t K,
                           const uint8_t* w_codes, const uint8_t* w_scales, float w_global,
                           double* y) {
    uint8_t* xc = (uint8_t*)malloc((size_t)M * (size_t)K / 2);
    uint8_t* xs = (uint8_t*)malloc((size_t)M * (size_t)K / 16);
    float* xd = (float*)malloc(sizeof(float) * (size_t)M * (size_t)K);
    float* wd = (float*)malloc(sizeof(float) * (size_t)N * (size_t)K);
    orc_quantize(x, M, K, input_scale, xc, xs);
    orc_dequantize(xc, xs, input_scale, M, K, xd, NULL);
    orc_dequantize(w_codes, w_scales, w_global, N, K, wd, NULL);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) acc += (double)wd[n * K + k] * (double)xd[m * K + k];
            y[m * N + n] = acc;
        }
    free(xc);
    free(xs);
    free(xd);
    free(wd);
}

/* ---------------------------------------------------------------------- */
/* Routed-expert MoE layer with NVFP4 experts                              */
/* ([P2] intro: 256 routed experts, 8 per token, hidden 6144;              */
/*  [P2] "Quantization recipe": experts in NVFP4)                           */
/* ---------------------------------------------------------------------- */

/* For every token t and slot j (expert e = ids[t, j], gate weight w[t, j]):
 *   x^   = x_t                                   (mode 0, W4A16)
 *        = deq(quantize(x_t, a13[e]))            (mode 1, W4A4, static scale)
 *   g, u = rows [0, I) and [I, 2I) of W13_e^ . x^   (fp64)
 *   h    = bf16(silu(g) * u),  silu(z) = z / (1 + exp(-z))
 *   h^   = h (mode 0)  or  deq(quantize(h, a2[e])) (mode 1)
 *   y    = W2_e^ . h^                             (fp64)
 *   out[t] = sum_j w[t, j] * y   (fp64, j in order)
 * Weights per expert: w13 [E, 2I, H] and w2 [E, H, I] NVFP4 with one global
 * scale per expert tensor.  h_out (optional) receives h as bf16 [T*k, I].
 * Each expert is dequantized once, only if some token uses it.
 *
 * Optional bf16 LoRA overlay on the experts ([P1] "Going deeper" ->
 * the rollout-engine passage: rank-64 bf16 LoRA on the MLP, applied to the
 * NVFP4 routed experts by a non-fused MoE-LoRA path, with one LoRA-A shared
 * by all experts and a LoRA-B per expert).  Rank r, multiplier `scale`:
 *   z13 = bf16(A13 . x_t)              A13 bf16 [r, H]   (bf16 x, both modes)
 *   g, u += scale * (B13_e . z13)      B13 bf16 [E, 2I, r], gate rows first
 *   z2  = bf16(A2 . h)                 A2  bf16 [r, I]   (bf16 h, both modes)
 *   y   += scale * (B2_e . z2)         B2  bf16 [E, H, r]
 * each dot product in fp64; a projection whose A (and B) is NULL has no
 * adapter.  The delta is added before the activation (gate/up) and before
 * the weighted combine (down). */
ORC_API void orc_moe_lora(int64_t T, int64_t E, int64_t topk, int64_t H, int64_t I, int32_t mode,
                          const uint16_t* x, const int32_t* ids, const float* w,
                          const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_global,
                          const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_global,
                          const float* a13, const float* a2, int64_t rank, float scale,
                          const uint16_t* lora_a13, const uint16_t* lora_b13, const uint16_t* lora_a2,
                          const uint16_t* lora_b2, double* out, uint16_t* h_out) {
    const int64_t slots = T * topk;
    for (int64_t i = 0; i < T * H; i++) out[i] = 0.0;
    double* y_all = (double*)calloc((size_t)slots * (size_t)H, sizeof(double));
    float* w13d = (float*)malloc(sizeof(float) * (size_t)(2 * I) * (size_t)H);
    float* w2d = (float*)malloc(sizeof(float) * (size_t)H * (size_t)I);
    for (int64_t e = 0; e < E; e++) {
        int used = 0;
        for (int64_t p = 0; p < slots; p++)
            if (ids[p] == e) { used = 1; break; }
        if (!used) continue;
        orc_dequantize(w13_codes + e * (2 * I) * (H / 2), w13_scales + e * (2 * I) * (H / 16),
                       w13_global[e], 2 * I, H, w13d, NULL);
        orc_dequantize(w2_codes + e * H * (I / 2), w2_scales + e * H * (I / 16), w2_global[e], H, I,
                       w2d, NULL);
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t p = 0; p < slots; p++) {
            if (ids[p] != e) continue;
            const int64_t t = p / topk;
            float* xh = (float*)malloc(sizeof(float) * (size_t)H);
            float* hh = (float*)malloc(sizeof(float) * (size_t)I);
            uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
            if (mode == 1) {
                uint8_t* qc = (uint8_t*)malloc((size_t)H / 2);
                uint8_t* qs = (uint8_t*)malloc((size_t)H / 16);
                orc_quantize(x + t * H, 1, H, a13[e], qc, qs);
                orc_dequantize(qc, qs, a13[e], 1, H, xh, NULL);
                free(qc);
                free(qs);
            } else {
                for (int64_t k = 0; k < H; k++) xh[k] = orc_bf16_to_f32(x[t * H + k]);
            }
            float* z = (float*)malloc(sizeof(float) * (size_t)(rank > 0 ? rank : 1));
            if (lora_a13) {
                for (int64_t q = 0; q < rank; q++) {
                    double acc = 0.0;
                    for (int64_t k = 0; k < H; k++)
                        acc += (double)orc_bf16_to_f32(lora_a13[q * H + k]) *
                               (double)orc_bf16_to_f32(x[t * H + k]);
                    z[q] = orc_bf16_to_f32(orc_f64_to_bf16(acc));
                }
            }
            for (int64_t i = 0; i < I; i++) {
                double g = 0.0, u = 0.0;
                for (int64_t k = 0; k < H; k++) {
                    g += (double)w13d[i * H + k] * (double)xh[k];
                    u += (double)w13d[(I + i) * H + k] * (double)xh[k];
                }
                if (lora_a13) {
                    const uint16_t* bg = lora_b13 + (e * 2 * I + i) * rank;
                    const uint16_t* bu = lora_b13 + (e * 2 * I + I + i) * rank;
                    double dg = 0.0, du = 0.0;
                    for (int64_t q = 0; q < rank; q++) {
                        dg += (double)orc_bf16_to_f32(bg[q]) * (double)z[q];
                        du += (double)orc_bf16_to_f32(bu[q]) * (double)z[q];
                    }
                    g += (double)scale * dg;
                    u += (double)scale * du;
                }
                double hv = g / (1.0 + exp(-g)) * u;
                hb[i] = orc_f64_to_bf16(hv);
            }
            if (h_out)
                for (int64_t i = 0; i < I; i++) h_out[p * I + i] = hb[i];
            if (mode == 1) {
                uint8_t* qc = (uint8_t*)malloc((size_t)I / 2);
                uint8_t* qs = (uint8_t*)malloc((size_t)I / 16);
                orc_quantize(hb, 1, I, a2[e], qc, qs);
                orc_dequantize(qc, qs, a2[e], 1, I, hh, NULL);
                free(qc);
                free(qs);
            } else {
                for (int64_t i = 0; i < I; i++) hh[i] = orc_bf16_to_f32(hb[i]);
            }
            if (lora_a2) {
                for (int64_t q = 0; q < rank; q++) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < I; i++)
                        acc += (double)orc_bf16_to_f32(lora_a2[q * I + i]) * (double)orc_bf16_to_f32(hb[i]);
                    z[q] = orc_bf16_to_f32(orc_f64_to_bf16(acc));
                }
            }
            for (int64_t n = 0; n < H; n++) {
                double acc = 0.0;
                for (int64_t i = 0; i < I; i++) acc += (double)w2d[n * I + i] * (double)hh[i];
                if (lora_a2) {
                    const uint16_t* bn = lora_b2 + (e * H + n) * rank;
                    double d = 0.0;
                    for (int64_t q = 0; q < rank; q++) d += (double)orc_bf16_to_f32(bn[q]) * (double)z[q];
                    acc += (double)scale * d;
                }
                y_all[p * H + n] = acc;
            }
            free(z);
            free(xh);
            free(hh);
            free(hb);
        }
    }
    for (int64_t t = 0; t < T; t++)
        for (int64_t j = 0; j < topk; j++) {
            const double wt = (double)w[t * topk + j];
            for (int64_t n = 0; n < H; n++) out[t * H + n] += wt * y_all[(t * topk + j) * H + n];
        }
    free(y_all);
    free(w13d);
    free(w2d);
}

/* The MoE layer without an adapter. */
ORC_API void orc_moe(int64_t T, int64_t E, int64_t topk, int64_t H, int64_t I, int32_t mode,
                     const uint16_t* x, const int32_t* ids, const float* w,
                     const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_global,
                     const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_global,
                     const float* a13, const float* a2, double* out, uint16_t* h_out) {
    orc_moe_lora(T, E, topk, H, I, mode, x, ids, w, w13_codes, w13_scales, w13_global, w2_codes, w2_scales,
                 w2_global, a13, a2, 0, 0.0f, NULL, NULL, NULL, NULL, out, h_out);
}
