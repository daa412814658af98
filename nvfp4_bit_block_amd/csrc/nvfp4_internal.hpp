// nvfp4_internal.hpp -- host-side launchers shared between the C ABI and the
// kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------- quantize --

// Number of workgroups of the dynamic-mode amax pass for n elements.
int amax_grid(int64_t n);

// Where the per-16-block global scale of a quantize pass comes from.
enum class ScaleMode : int {
    kDynamic = 0,  // fl(amax / 2688) from the per-workgroup maxima `partial`
    kStatic = 1,   // *sg_ptr
    kGrouped = 2,  // sg_group[row_group[row]] (per-row static scale)
};

struct PackArgs {
    const uint16_t* x = nullptr;    // bf16 source
    int64_t rows = 0, cols = 0;     // output shape (cols % 16 == 0)
    const int32_t* src_row = nullptr;  // optional gather: source row = src_row[r] / src_div
    int32_t src_div = 1;
    const int32_t* rows_valid = nullptr;  // optional device count: rows >= *rows_valid are skipped
    ScaleMode mode = ScaleMode::kStatic;
    const uint32_t* partial = nullptr;
    int npartial = 0;
    const float* sg_ptr = nullptr;
    const float* sg_group = nullptr;
    const int32_t* row_group = nullptr;
    uint8_t* codes = nullptr;       // [rows, cols/2] (optional when xhat is set)
    uint8_t* scales = nullptr;      // [rows, cols/16]
    float* global_out = nullptr;    // optional: the Sg used (uniform modes only)
    // Optional decoded output [rows, cols]: the exact products q * s of each
    // element (no global scale), as f16 or bf16 (both represent them exactly).
    uint16_t* xhat = nullptr;
    bool xhat_bf16 = false;
    // kGrouped with n_groups > 0: when the n_groups scales sg_group[0 ..
    // n_groups) are all bitwise equal, rows 0 .. shared_rows - 1 of x are
    // quantized instead, ungathered, under sg_group[0] (output row r from
    // source row r); every workgroup takes the same choice and workgroup 0
    // stores it in *shared_out (1 shared, 0 per-row scales).
    int32_t n_groups = 0;
    int64_t shared_rows = 0;
    int32_t* shared_out = nullptr;
};

hipError_t launch_amax_partial(const uint16_t* x, int64_t n, uint32_t* partial, int grid,
                               hipStream_t stream);

// The no-alloc quantize keeps its pass-1 partial maxima in a static device
// array of kNoAllocPartials entries per GPU (quantize.hip); *out receives its
// device address on the device of `stream` (the current device for NULL).
constexpr int kNoAllocPartials = 1024;
hipError_t noalloc_partials(hipStream_t stream, uint32_t** out);
hipError_t launch_quantize_pack(const PackArgs& a, hipStream_t stream);

// y = bf16(fl(fl(q*s) * Sg)); Sg = *sg_ptr, or `sg_const` when sg_ptr is null.
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* sg_ptr,
                             float sg_const, int64_t rows, int64_t cols, uint16_t* y,
                             hipStream_t stream);

// Packed codes + scales [rows, cols] -> the exact products q * s (no global
// scale), f16 or bf16 [rows, cols].
hipError_t launch_expand_qs(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                            uint16_t* out, bool bf16, hipStream_t stream);

// Columnwise NVFP4 (transpose.hip): x bf16 [rows, cols] -> codes_t [cols,
// rows/2] and scales_t [cols, rows/16], the rowwise quantization of x^T.
// rows % 16 == 0, cols % 8 == 0.  Modes kDynamic (partials from
// launch_amax_partial over x) and kStatic (*sg_ptr).
hipError_t launch_quantize_cols(const uint16_t* x, int64_t rows, int64_t cols, ScaleMode mode,
                                const uint32_t* partial, int npartial, const float* sg_ptr, uint8_t* codes_t,
                                uint8_t* scales_t, float* global_out, hipStream_t stream);

// Rowwise NVFP4 [rows, cols] -> bf16 y_t [cols, rows] = transpose of the
// dequantized tensor.  rows % 8 == 0, cols % 16 == 0.
hipError_t launch_dequantize_t(const uint8_t* codes, const uint8_t* scales, const float* sg_ptr, int64_t rows,
                               int64_t cols, uint16_t* y_t, hipStream_t stream);

// -------------------------------------------------------------------- GEMV --

// y[m, n] = bf16(scale * sum_k s*q*x), scale = *g0 * (g1 ? *g1 : 1).
hipError_t launch_gemv_w4a16(const uint16_t* x, int M, int64_t N, int64_t K, const uint8_t* wc,
                             const uint8_t* ws, const float* g0, const float* g1, uint16_t* y,
                             hipStream_t stream);

// W4A4 at M = 1 in one launch: the GEMV quantizes the bf16 activation x
// under *input_scale in registers (same codes and scales as
// launch_quantize_pack in static mode) and multiplies with the exact q * s;
// y = bf16(*w_global * *input_scale * sum).  Available when
// gemv_quantizes_activation(M, K); hipErrorNotSupported otherwise.
bool gemv_quantizes_activation(int M, int64_t K);
hipError_t launch_gemv_w4a4(const uint16_t* x, int M, int64_t N, int64_t K, const uint8_t* wc,
                            const uint8_t* ws, const float* w_global, const float* input_scale,
                            uint16_t* y, hipStream_t stream);

// W4A4 GEMV on a pre-packed activation (codes [M, K/2], scales [M, K/16],
// global scale a_global), decoded in registers; for the M, K of
// gemv_takes_packed(M, K), hipErrorNotSupported otherwise.
bool gemv_takes_packed(int M, int64_t K);
hipError_t launch_gemv_w4a4_packed(const uint8_t* a_codes, const uint8_t* a_scales, int M, int64_t N, int64_t K,
                                   const uint8_t* wc, const uint8_t* ws, const float* w_global,
                                   const float* a_global, uint16_t* y, hipStream_t stream);

// -------------------------------------------------------------------- GEMM --

// A operand formats: bf16 values, or f16 values that are the exact products
// q * s of an NVFP4 encoding.
enum class AFmt : int { kBf16 = 0, kF16 = 2 };
enum class Epi : int {
    kStoreBf16 = 0,   // y = bf16(acc * scale)
    kPartialF32 = 1,  // partial[split] = acc (split-K, reduced later)
    kMoeGateUp = 2,   // h = bf16(silu(g*scale) * (u*scale)) (and its NVFP4 q * s with out_q)
    kMoeDown = 3,     // Y = acc * scale (fp32)
    kMoeGateUpLora = 4,  // kMoeGateUp with the LoRA overlay added before the activation
    kMoeDownLora = 5,    // kMoeDown with the LoRA overlay
};

struct GemmArgs {
    // A operand: 16-bit [*, K] rows (optionally gathered).
    const void* a = nullptr;
    const int32_t* a_rows = nullptr;  // gather: A row of output row r = a_rows[r] / a_div
    int32_t a_div = 1;
    const int32_t* a_rows_on = nullptr;  // optional device flag: the gather applies only when it is nonzero
    int64_t a_src_rows = 0;           // bf16 A: rows of the source tensor
    const float* a_global = nullptr;  // per group (or [1]); null = 1
    // B operand: NVFP4 [N, K] per group
    const uint8_t* b_codes = nullptr;
    const uint8_t* b_scales = nullptr;
    const float* b_global = nullptr;  // per group (or [1])
    int64_t M = 0, N = 0, K = 0;
    // grouping (MoE): rows of group e are [row_off[e], row_off[e+1]); its
    // m-tiles are [tile_off[e], tile_off[e+1]); a/b pointers advance per group
    const int32_t* row_off = nullptr;
    const int32_t* tile_off = nullptr;
    int32_t groups = 0;
    int32_t grouped_ntiles = 0;  // set by the launcher
    // output
    void* out = nullptr;
    int64_t ldo = 0;
    // gate/up epilogues only: when out_q is set, h is also NVFP4-quantized
    // under the per-group static scale q_global[group] (blocks of 16 along
    // the row) and written to out_q [*, ldo] as the exact f16 products q * s,
    // the operand of the down projection; out (bf16 h) may then be null.
    uint16_t* out_q = nullptr;
    const float* q_global = nullptr;
    int32_t ksplit = 1;
    // stream-K (ungrouped kPartialF32, ksplit 1): the mtiles ntiles (K / 64)
    // K steps, tile after tile, are dealt evenly to sk_wgs workgroups; the
    // part of tile t done by workgroup w goes to partial slot w - first(t)
    // (first(t): the workgroup holding the tile's first step), summed by
    // launch_streamk_reduce; a tile done whole by one workgroup is written
    // straight to sk_y (bf16 [M, ldo], scaled) and the finish skips it.
    // 0: the ksplit layout.
    int32_t sk_wgs = 0;
    uint16_t* sk_y = nullptr;
    int64_t half_n = 0;  // gate/up epilogue: I (the up rows start at I)
    // LoRA overlay (the kMoe*Lora epilogues, ksplit 1): the
    // epilogue value of (row, col) becomes
    //   acc * globals + lora_scale * sum_q Z[zrow, q] * Bg[col, q]
    // with Z bf16 [*, lora_rank] (zrow = lora_rows ? lora_rows[row] / lora_div
    // : row) and Bg bf16 [N, lora_rank] the group's slice of lora_b.
    const uint16_t* lora_z = nullptr;
    const int32_t* lora_rows = nullptr;
    int32_t lora_div = 1;
    const uint16_t* lora_b = nullptr;
    int32_t lora_rank = 0;  // a multiple of 8
    float lora_scale = 0.0f;
};

// GEMM tiles with a 16-bit A operand (gemm_a16.hip): f16 products q * s
// (W4A4) or bf16 activations (W4A16); NVFP4 B.  Workgroup tile rows x cols
// and the per-wave tile.
enum class A16Tile : int {
    k256x256_w128x64 = 0,
    k128x128_w64x64 = 5,
    k128x128_w32x64 = 6,
    k64x256_w64x64 = 7,
    k32x256_w32x64 = 8,
    k192x128_w96x64 = 9,
};
int a16_tile_rows(A16Tile t);
// Each operand of launch_gemm_a16 is addressed through one buffer resource
// and must span fewer bytes than this.
constexpr int64_t kMaxOperandBytes = (int64_t)1 << 31;
int a16_tile_cols(A16Tile t);
hipError_t launch_gemm_a16(const GemmArgs& g, AFmt afmt, Epi epi, A16Tile tile, int grid_m,
                           hipStream_t stream);

// Rank-r projection of LoRA's shared A (lora.hip): Z [rows, R] =
// bf16(X [rows, K] * A [R, K]^T) with fp32 accumulation; K % 64 == 0,
// R % 8 == 0, R <= 128.
hipError_t launch_lora_a(const uint16_t* x, int64_t rows, int64_t K, const uint16_t* a, int R, uint16_t* z,
                         hipStream_t stream);
// y[m, n] = bf16(scale * sum_s partial[s][m][n]), scale = *g0 * (g1 ? *g1 : 1)
hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N,
                                const float* g0, const float* g1, uint16_t* y, hipStream_t stream);
// Stream-K on the ungrouped tile `tile`: the most partial slots one tile
// takes with `wgs` workgroups (the partial buffer holds that many [M, N]
// slots), or 0 when wgs exceeds the K steps of the problem.
int streamk_slots(int64_t M, int64_t N, int64_t K, A16Tile tile, int wgs);
// The stream-K finish: y[m, n] = bf16(scale * sum over the slots of the tile
// holding (m, n), in slot order), scale as for launch_splitk_reduce; tiles
// of one slot were written by the GEMM itself and are left alone.
hipError_t launch_streamk_reduce(const float* partial, int64_t M, int64_t N, int64_t K, A16Tile tile, int wgs,
                                 const float* g0, const float* g1, uint16_t* y, hipStream_t stream);

// ------------------------------------------------------- small-batch stream --

// Activation operand of the weight-streaming GEMM (gemm_stream.hip).
enum class SAct : int {
    kBf16 = 0,    // bf16 [M, K] (W4A16; weights decoded to bf16 q * s)
    kF16 = 1,     // f16 [M, K]: the exact products q * s of an NVFP4 activation
    kPacked = 2,  // NVFP4 codes [M, K/2] + E4M3 scale bytes [M, K/16]
    kQuant = 3,   // bf16 [M, K], quantized in registers under *a_global (static)
    kPackedLds = 4,  // as kPacked, streamed through LDS with the weights (M > 16)
    kBf16Lds = 5,    // as kBf16, streamed through LDS with the weights (long rows)
};

struct StreamArgs {
    const void* a = nullptr;            // see SAct
    const uint8_t* a_scales = nullptr;  // kPacked: scale bytes [M, K/16]
    const float* a_global = nullptr;    // activation global scale (kQuant: the static input scale); null = 1
    const uint8_t* b_codes = nullptr;   // weight NVFP4 [N, K]
    const uint8_t* b_scales = nullptr;
    const float* b_global = nullptr;
    int64_t M = 0, N = 0, K = 0;
    int32_t ksplit = 1;                 // K ranges of krange (the last may be shorter)
    int64_t krange = 0;                 // a multiple of 128
    void* out = nullptr;                // ksplit 1: bf16 Y [M, N]; else fp32 partials [ksplit, M, N]
};

// Y = A W^T for 1 <= M <= 16 mb on a grid of ceil(N / (16 nb)) x ksplit
// workgroups of 8 waves, nb in {2, 4}, mb in {1, 2, 4} (kPackedLds: 2, 4
// or 8, the last on 512-K ring stages; kBf16Lds: 1, 2 or 4, the last two on
// 512-K ring stages); K % 128 == 0 and
// N * K / 2 < 2^31.  Each K range may hold at most stream_max_chunks(am, mb)
// chunks of 1024 (rounded up to a power of two); hipErrorInvalidValue
// otherwise.
int stream_max_chunks(SAct am, int mb);
hipError_t launch_gemm_stream(const StreamArgs& g, SAct am, int nb, int mb, hipStream_t stream);

// --------------------------------------------------------------------- MoE --

// Routing: per-expert row offsets row_off [E + 1] and bm-row tile offsets
// tile_off [E + 1], the slot of each expert row perm [slots], the row of each
// slot inv [slots] (-1 for an id outside [0, E)) and the expert of each row
// pos_group [slots].  `scratch` holds moe_route_scratch_bytes(slots, E) bytes
// of per-workgroup counts.  E <= 4096.
size_t moe_route_scratch_bytes(int64_t slots, int32_t E);
hipError_t launch_moe_route(const int32_t* ids, int64_t slots, int32_t E, int32_t bm,
                            int32_t* row_off, int32_t* tile_off, int32_t* perm, int32_t* inv,
                            int32_t* pos_group, int32_t* scratch, hipStream_t stream);

hipError_t launch_moe_combine(const float* Y, const int32_t* inv, const float* w, int64_t T,
                              int32_t topk, int64_t H, uint16_t* out, hipStream_t stream);

}  // namespace nvfp4
