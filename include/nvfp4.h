/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 library.
 *
 * NVFP4 as used here ("Getting GLM-5.2 NVFP4 Post-Training off the ground",
 * section "Going deeper: why a 4-bit weight needs two copies on B200"; the
 * "GLM-5.2-NVFP4" model card, "Quantization recipe"; the
 * "vroomfondel/glm-5.2-reap-504B-v2-W4A4" model card, "How it was produced"):
 *   - every element is a 4-bit E2M1 code (sign bit 3; magnitudes
 *     0, .5, 1, 1.5, 2, 3, 4, 6), two codes per byte, the even element in
 *     the low nibble;
 *   - every run of 16 consecutive elements along a row (the contraction axis)
 *     shares one E4M3 ("fn", max 448) scale byte; scales are stored linearly,
 *     [rows, cols/16] row-major;
 *   - the tensor carries one fp32 global scale; from a bf16 tensor it is
 *     amax / (6 * 448) (the checkpoint's weight_scale_2); for activations of
 *     the W4A4 path it is a static per-tensor input_scale chosen ahead of time.
 *   - A value decodes as q * s * Sg.  Encoding rounds to nearest, ties to the
 *     even code, saturating at 6 (elements) and 448 (scales), in this fp32
 *     order: t = 6*Sg; per block s8 = E4M3(bmax / t), s = value(s8);
 *     per element d = s*Sg, code = sign(x) | E2M1(|x| / d) (0 when d == 0).
 *
 * Conventions for every entry point:
 *   - Tensors are device pointers to contiguous row-major storage; bf16 is
 *     passed as uint16_t bit patterns, codes and scale bytes as uint8_t.
 *     Tensor base pointers (bf16, codes, scale bytes, outputs, workspace) must
 *     be 16-byte aligned; fp32 scale pointers and the MoE routing arrays
 *     (int32 ids, fp32 weights, per-expert fp32 scales) 4-byte aligned
 *     (ALIGN otherwise).
 *   - Scalars that live with the tensors (global scales, input_scale) are
 *     device pointers to fp32, so no call reads device memory on the host.
 *   - The caller allocates and frees every buffer, workspace included; the
 *     library allocates no memory and keeps no device state between calls,
 *     except the 4 KB static scratch array of nvfp4_quantize_noalloc.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without waiting for it.  Outputs must not alias
 *     inputs.  Calls on the same stream are ordered; a workspace must not be
 *     shared by calls that can run concurrently.
 *   - Every argument check except NVFP4_ERR_HIP happens on the host before
 *     any HIP call, so invalid arguments never reach the device.  Checks run
 *     in this order: shape (SHAPE, then UNSUPPORTED), zero size, pointers
 *     (NULL_ARG, ALIGN), workspace.  A zero-sized problem (rows, M, N or T
 *     equal to 0) with valid dimensions is a successful no-op, whatever its
 *     pointers.
 *   - Device-side preconditions (not checked): inputs are finite; static
 *     scales are finite and > 0; routing ids outside [0, E) are skipped.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int32_t entry point. */
#define NVFP4_OK 0
#define NVFP4_ERR_NULL_ARG 1    /* a required pointer is NULL */
#define NVFP4_ERR_SHAPE 2       /* negative dimension, K/cols not a multiple of 16, ... */
#define NVFP4_ERR_ALIGN 3       /* a tensor pointer is not 16-byte aligned */
#define NVFP4_ERR_UNSUPPORTED 4 /* valid NVFP4 problem outside the kernels provided */
#define NVFP4_ERR_WORKSPACE 5   /* workspace NULL or smaller than the query says */
#define NVFP4_ERR_HIP 6         /* a HIP launch failed; see nvfp4_last_error() */

/* Library version, major*10000 + minor*100 + patch. */
int32_t nvfp4_version(void);

/* Static text for a status code. */
const char* nvfp4_status_string(int32_t status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* nvfp4_last_error(void);

/* ------------------------------------------------------------------------
 * Quantize  (model card "vroomfondel/glm-5.2-reap-504B-v2-W4A4", "How it was
 * produced": data-free weight packing with weight_scale_2 = amax/(6*448);
 * static input_scale for activations.)
 *
 * x            bf16 [rows, cols], cols % 16 == 0.
 * static_scale NULL: dynamic mode, Sg = fl(amax(|x|) / 2688) computed on the
 *              device (two passes: per-workgroup maxima into `workspace`,
 *              then scales and codes).  Non-NULL: device fp32 Sg used as is
 *              (one pass; the W4A4 input_scale path); workspace unused.
 * codes        out uint8 [rows, cols/2]; scales out uint8 [rows, cols/16].
 * global_scale out device fp32 [1]: the Sg that was used.
 * workspace    device scratch of nvfp4_quantize_workspace_size(rows, cols)
 *              bytes (dynamic mode only; may be NULL when that size is 0).
 * Output is bit-identical to the plain CPU definition above.
 * ------------------------------------------------------------------------ */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols);
int32_t nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, const float* static_scale,
                       uint8_t* codes, uint8_t* scales, float* global_scale, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Quantize without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and checks as nvfp4_quantize
 * without the workspace; bit-identical output.
 *
 * Dynamic mode keeps its pass-1 partial maxima in a static device array of
 * 1024 uint32 (4 KB) that each GPU holds from the first call until the
 * process ends (amax_grid never needs more than 768 of them, so no shape the
 * dynamic quantize accepts is refused for its size; a rows * cols product
 * past 2^62 is UNSUPPORTED).  The first call on a device resolves the array's
 * address there (hipGetSymbolAddress, with the stream's device current); the
 * call never allocates or frees memory.  Every call on a GPU shares that
 * GPU's array: calls that can overlap on one GPU (different streams, no
 * ordering between them) race and must not be issued.  Static mode uses no
 * scratch at all.
 * ------------------------------------------------------------------------ */
int32_t nvfp4_quantize_noalloc(const uint16_t* x, int64_t rows, int64_t cols, const float* static_scale,
                               uint8_t* codes, uint8_t* scales, float* global_scale, void* stream);

/* ------------------------------------------------------------------------
 * Dequantize  ("Getting GLM-5.2 NVFP4 Post-Training off the ground", "Going
 * deeper": dequantize the rowwise copy to bf16.)
 * y[r, c] = bf16_rne(fl(fl(q * s) * Sg)); codes [rows, cols/2], scales
 * [rows, cols/16], global_scale device fp32 [1], y bf16 [rows, cols].
 * ------------------------------------------------------------------------ */
int32_t nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                         int64_t rows, int64_t cols, uint16_t* y, void* stream);

/* ------------------------------------------------------------------------
 * The Dgrad layouts ("Getting GLM-5.2 NVFP4 Post-Training off the ground",
 * "Going deeper" and "The bottom line"): Dgrad, dX = dY * W, contracts the
 * weight over its output axis, and NVFP4 blocks must run along the
 * contraction axis, so the rowwise copy's scales cannot serve it.
 *
 * nvfp4_quantize_columnwise: the columnwise copy, i.e. the NVFP4 quantization
 * of x^T computed from the full-precision x (blocks of 16 along rows, same
 * global scale and block rule as nvfp4_quantize, dynamic or static).
 * x bf16 [rows, cols] -> codes_t [cols, rows/2], scales_t [cols, rows/16],
 * *global_scale.  rows % 16 == 0 (else SHAPE), cols % 8 == 0 and rows <=
 * 65535 * 128 (else UNSUPPORTED).  Workspace as nvfp4_quantize: nvfp4_quantize_workspace_size
 * (rows, cols) bytes in dynamic mode, none in static mode.  Bit-identical to
 * nvfp4_quantize of the transposed tensor.
 *
 * nvfp4_dequantize_transpose: the page's alternative, the rowwise copy
 * dequantized to bf16 and transposed on the fly for a bf16 Dgrad:
 * y_t[c, r] = bf16( fl(fl(q[r, c] * s[r, c/16]) * Sg) ), y_t bf16 [cols, rows]
 * (the transpose of nvfp4_dequantize's output, bit for bit).  cols % 16 == 0
 * (else SHAPE), rows % 8 == 0 and cols <= 65535 * 128 (else UNSUPPORTED).
 * No workspace.
 * ------------------------------------------------------------------------ */
int32_t nvfp4_quantize_columnwise(const uint16_t* x, int64_t rows, int64_t cols, const float* static_scale,
                                  uint8_t* codes_t, uint8_t* scales_t, float* global_scale, void* workspace,
                                  size_t workspace_bytes, void* stream);
int32_t nvfp4_dequantize_transpose(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                                   int64_t rows, int64_t cols, uint16_t* y_t, void* stream);

/* ------------------------------------------------------------------------
 * W4A16 decode GEMV  (model card "vroomfondel/glm-5.2-reap-504B-v2-W4A4",
 * "What this variant changes": batch-1 decode projections are weight-bandwidth
 * bound; "Kernel choice": the weight-only NVFP4 path.)
 * y[m, n] = bf16( Sg_w * sum_k s[n, k/16] * q[n, k] * x[m, k] ), fp32 accumulation.
 * x bf16 [M, K]; w_codes [N, K/2]; w_scales [N, K/16]; w_global device fp32
 * [1]; y bf16 [M, N].  1 <= M <= 8 and K % 32 == 0 (else UNSUPPORTED).
 * No workspace.
 * ------------------------------------------------------------------------ */
int32_t nvfp4_gemv_w4a16(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_codes,
                         const uint8_t* w_scales, const float* w_global, uint16_t* y, void* stream);

/* ------------------------------------------------------------------------
 * W4A4 GEMM, Fprop Y = X * W^T with K innermost on both operands ("Getting
 * GLM-5.2 NVFP4 Post-Training off the ground", "Going deeper" and "TN, NT, and
 * what actually binds"; model card "vroomfondel/glm-5.2-reap-504B-v2-W4A4",
 * "How it was produced" and "Kernel choice": static input_scale, no dynamic
 * activation quantization).
 * X bf16 [M, K] is quantized to NVFP4 under the device fp32 *input_scale
 * (same arithmetic as nvfp4_quantize in static mode), then
 * y[m, n] = bf16( input_scale * Sg_w * sum_b sx[m,b] sw[n,b] sum_{k in b} qx qw ),
 * fp32 accumulation.  w_* as in the GEMV; y bf16 [M, N].  K % 64 == 0, and
 * unless M <= 4 (or M <= 8 with K <= 4096 or K == 16384) the weight codes must span less
 * than 2 GiB (N * K / 2 < 2^31); else UNSUPPORTED.  Workspace: nvfp4_gemm_w4a4_workspace_size(M, N, K)
 * bytes (the quantized X, held as its exact products q * s in 16-bit form,
 * and the fp32 partial sums of a K split or, on long rows, of tiles whose K
 * range several workgroups share).
 * ------------------------------------------------------------------------ */
size_t nvfp4_gemm_w4a4_workspace_size(int64_t M, int64_t N, int64_t K);
int32_t nvfp4_gemm_w4a4(const uint16_t* x, const float* input_scale, int64_t M, int64_t N, int64_t K,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                        uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * W4A4 GEMM on a pre-packed NVFP4 activation: the serving split in which a
 * producer quantizes X once under the static input_scale (nvfp4_quantize in
 * static mode; model card "vroomfondel/glm-5.2-reap-504B-v2-W4A4", "How it
 * was produced": static input_scale, no dynamic activation quantization) and
 * the GEMM consumes codes and scales.
 * y[m, n] = bf16( a_global * Sg_w * sum_b sx[m,b] sw[n,b] sum_{k in b} qx qw ),
 * fp32 accumulation; identical to nvfp4_gemm_w4a4 on the X those codes came
 * from.  a_codes [M, K/2], a_scales [M, K/16], a_global device fp32 [1] (the
 * static scale the codes were made with); w_* as in the GEMV; y bf16 [M, N].
 * Same shape limits as nvfp4_gemm_w4a4.  Workspace:
 * nvfp4_gemm_w4a4_packed_workspace_size(M, N, K) bytes (the activation
 * expanded to its exact products q * s, and fp32 partial sums as for
 * nvfp4_gemm_w4a4).
 * ------------------------------------------------------------------------ */
size_t nvfp4_gemm_w4a4_packed_workspace_size(int64_t M, int64_t N, int64_t K);
int32_t nvfp4_gemm_w4a4_packed(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global, int64_t M,
                               int64_t N, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                               const float* w_global, uint16_t* y, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * W4A16 GEMM over any M: the weight-only path of the model card
 * "vroomfondel/glm-5.2-reap-504B-v2-W4A4", "Kernel choice", measured against
 * W4A4 across the batch sweep (that section compares the two kernel families
 * from batch 1 upward).  Same product as the GEMV,
 * y[m, n] = bf16( Sg_w * sum_k s[n, k/16] * q[n, k] * x[m, k] ), fp32
 * accumulation, with x bf16 [M, K] used as is (no activation quantization).
 * Small M runs the GEMV kernels; larger M runs MFMA tiles whose weight
 * operand is decoded to the exact bf16 values q * s.  K % 64 == 0, and when
 * the tiles run the weight codes must span less than 2 GiB; else UNSUPPORTED.
 * Workspace: nvfp4_gemm_w4a16_workspace_size(M, N, K) bytes (fp32 partial
 * sums as for nvfp4_gemm_w4a4; 0 when none are needed, and then workspace
 * may be NULL).
 * ------------------------------------------------------------------------ */
size_t nvfp4_gemm_w4a16_workspace_size(int64_t M, int64_t N, int64_t K);
int32_t nvfp4_gemm_w4a16(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_codes,
                         const uint8_t* w_scales, const float* w_global, uint16_t* y, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Routed-expert MoE layer with NVFP4 experts ("GLM-5.2-NVFP4" model card:
 * 256 routed experts, 8 per token, hidden 6144, experts quantized to NVFP4;
 * W4A4 variant as in "vroomfondel/glm-5.2-reap-504B-v2-W4A4").
 *
 * For each token t and slot j < top_k with expert e = topk_ids[t, j]:
 *   mode 0 (W4A16): x^ = x[t];  mode 1 (W4A4): x^ = NVFP4(x[t], a13_scale[e]).
 *   [g | u] = x^ * W13_e^T (gate rows 0..I-1, up rows I..2I-1 of W13_e);
 *   h = bf16(silu(g) * u);  mode 1: h^ = NVFP4(h, a2_scale[e]) else h^ = h;
 *   out[t] = bf16( sum_j topk_weights[t, j] * (h^ * W2_e^T) ), fp32, j in order.
 * x bf16 [T, H]; topk_ids int32 [T, top_k]; topk_weights fp32 [T, top_k];
 * w13_codes [E, 2I, H/2], w13_scales [E, 2I, H/16], w13_global fp32 [E];
 * w2_codes [E, H, I/2], w2_scales [E, H, I/16], w2_global fp32 [E];
 * a13_scale, a2_scale fp32 [E] (mode 1 only, else may be NULL); out bf16 [T, H].
 * H % 64 == 0 and I % 64 == 0, and every operand the grouped GEMMs read
 * below 2 GiB (T*H*2 for mode 0 or T*top_k*H*2 for mode 1, T*top_k*I*2,
 * the codes of one expert's W13 and W2); else UNSUPPORTED.  Routing,
 * grouping, both grouped GEMMs and the combine run on the device with no
 * host round trip.  Workspace: nvfp4_moe_workspace_size(p) bytes (routing
 * tables, h, the fp32 per-slot outputs and, for mode 1, the quantized
 * activations held as their exact products q * s in f16: one row per slot,
 * or one per token when all E values of a13_scale are bitwise equal, which
 * the device checks on every call; the output bits are the same either way).
 * ------------------------------------------------------------------------ */
typedef struct nvfp4_moe_problem {
    int64_t T;      /* tokens */
    int64_t E;      /* routed experts */
    int64_t top_k;  /* experts per token */
    int64_t H;      /* hidden size (GEMM1 K, GEMM2 N) */
    int64_t I;      /* expert intermediate size (GEMM1 N/2, GEMM2 K) */
    int32_t mode;   /* 0 = W4A16, 1 = W4A4 */
} nvfp4_moe_problem;

typedef struct nvfp4_moe_tensors {
    const uint16_t* x;
    const int32_t* topk_ids;
    const float* topk_weights;
    const uint8_t* w13_codes;
    const uint8_t* w13_scales;
    const float* w13_global;
    const uint8_t* w2_codes;
    const uint8_t* w2_scales;
    const float* w2_global;
    const float* a13_scale;
    const float* a2_scale;
    uint16_t* out;
} nvfp4_moe_tensors;

size_t nvfp4_moe_workspace_size(const nvfp4_moe_problem* p);
int32_t nvfp4_moe_grouped_gemm(const nvfp4_moe_problem* p, const nvfp4_moe_tensors* t, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The same layer with a bf16 LoRA overlay on the routed experts ("Getting
 * GLM-5.2 NVFP4 Post-Training off the ground", "Going deeper": a rank-64
 * bf16 LoRA on the MLP of an NVFP4 base, applied to the routed experts by a
 * non-fused MoE-LoRA path, with one LoRA-A shared by all experts and one
 * LoRA-B per expert).  With r = rank and c = scale:
 *   z13 = bf16(x[t] * a13^T)   (the bf16 token, in both modes)
 *   [g | u] += c * (z13 * b13_e^T)          before the activation
 *   z2  = bf16(h * a2^T)       (the bf16 h, in both modes)
 *   y_slot  += c * (z2 * b2_e^T)            before the weighted combine
 * products accumulated in fp32.  a13 bf16 [r, H] and b13 bf16 [E, 2I, r]
 * (gate rows first, as in W13) adapt the gate/up projection; a2 bf16 [r, I]
 * and b2 bf16 [E, H, r] the down projection.  Either pair may be NULL (no
 * adapter there); a pair with one NULL member is NULL_ARG.  The adapter
 * tensors are 16-byte aligned (ALIGN).  rank <= 0 is SHAPE; rank % 8 != 0 or
 * rank > 128 is UNSUPPORTED.  lora == NULL runs nvfp4_moe_grouped_gemm.
 * Workspace: nvfp4_moe_lora_workspace_size(p, lora) bytes (the layer's
 * workspace plus z13 [T, r] and z2 [T*top_k, r] in bf16).
 * ------------------------------------------------------------------------ */
typedef struct nvfp4_moe_lora {
    int64_t rank;          /* r */
    float scale;           /* c, multiplies the adapter's product (alpha / r) */
    const uint16_t* a13;   /* bf16 [r, H] or NULL */
    const uint16_t* b13;   /* bf16 [E, 2I, r] or NULL */
    const uint16_t* a2;    /* bf16 [r, I] or NULL */
    const uint16_t* b2;    /* bf16 [E, H, r] or NULL */
} nvfp4_moe_lora;

size_t nvfp4_moe_lora_workspace_size(const nvfp4_moe_problem* p, const nvfp4_moe_lora* lora);
int32_t nvfp4_moe_grouped_gemm_lora(const nvfp4_moe_problem* p, const nvfp4_moe_tensors* t,
                                    const nvfp4_moe_lora* lora, void* workspace, size_t workspace_bytes,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
