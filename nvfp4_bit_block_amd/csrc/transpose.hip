// transpose.hip -- the two layouts a linear layer's weight needs in training
// ("Getting GLM-5.2 NVFP4 Post-Training off the ground", "Going deeper" and
// "The bottom line"): Fprop contracts W [out, in] over in, Dgrad (dX = dY W)
// over out.  NVFP4 blocks run along the contraction axis, so the Dgrad operand
// is either a second, columnwise quantization (blocks of 16 along out, scales
// computed from the full-precision weight, not from the rowwise scales) or
// the rowwise copy dequantized to bf16 and transposed on the fly, the
// memory-for-compute trade the page makes.
//
//   k_quantize_cols   x bf16 [R, C] -> NVFP4 of x^T: codes [C, R/2],
//                     scales [C, R/16], blocks of 16 along R, with the same
//                     global scale and block rule as the rowwise quantizer.
//   k_dequant_t       rowwise NVFP4 [R, C] -> bf16 y^T [C, R],
//                     y = bf16(fl(fl(q s) Sg)) as in the dequantizer.
//
// Both stage a tile through LDS so that global reads and writes stay
// row-contiguous on both sides of the transpose.
#include "nvfp4_device.hpp"
#include "nvfp4_encode.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------- columnwise quantize --
// Tile: 128 rows x 64 columns of x.  Load: 16 bytes (8 columns) per thread,
// 8 threads per row.  LDS holds the tile row-major, 32 words (64 columns) per
// row, with word w of row r stored at w ^ (8 ((r / 16) mod 4)): a wave's
// encode reads (8 column pairs x 8 row blocks) then fall on 32 different
// banks, and the 16-byte row pieces stay aligned for 16-byte stores.
// Encode: thread t owns the column pair (2 (t / 8), +1) and the 16-row block
// t % 8; it reads 16 words (both columns of one row each), regroups them
// into bf16 pairs along R, and encodes one block per column.
constexpr int kQR = 128, kQC = 64;
constexpr int kQWords = kQC / 2;    // words per LDS row

__device__ __forceinline__ int qc_word(int r, int w) { return r * kQWords + (w ^ (((r >> 4) & 3) << 3)); }

template <ScaleMode MODE>
__global__ __launch_bounds__(kThreads) void k_quantize_cols(const uint16_t* __restrict__ x, int64_t R,
                                                            int64_t C, const uint32_t* __restrict__ partial,
                                                            int npartial, const float* __restrict__ sg_ptr,
                                                            uint8_t* __restrict__ codes_t,
                                                            uint8_t* __restrict__ scales_t,
                                                            float* __restrict__ global_out) {
    __shared__ __align__(16) uint32_t tile[kQR * kQWords];
    float Sg;
    if constexpr (MODE == ScaleMode::kDynamic) {
        uint32_t m = 0;
        for (int i = threadIdx.x; i < npartial; i += kThreads) m = max(m, partial[i]);
        m = wave_max_u32(m);
        __shared__ uint32_t red[kThreads / kWave];
        if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
        __syncthreads();
        m = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) m = max(m, red[w]);
        Sg = bf16_to_f32(m) / 2688.0f;
    } else {
        Sg = *sg_ptr;
    }
    if (global_out != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *global_out = Sg;
    const float t = 6.0f * Sg;

    const int64_t r0 = (int64_t)blockIdx.y * kQR, c0 = (int64_t)blockIdx.x * kQC;
    // load (columns past C read as zero; rows past R are never encoded)
#pragma unroll
    for (int pass = 0; pass < kQR / 32; ++pass) {
        const int lr = pass * 32 + (threadIdx.x >> 3), lc = (threadIdx.x & 7) * 8;
        const int64_t r = r0 + lr, c = c0 + lc;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < R && c < C) v = load_nt16(x + r * C + c);   // C % 8 == 0
        *reinterpret_cast<uint4*>(tile + qc_word(lr, lc / 2)) = v;
    }
    __syncthreads();

    const int cp = threadIdx.x >> 3, blk = threadIdx.x & 7;
    const int64_t rb = r0 + 16 * blk;      // first row of the block
    const int64_t c = c0 + 2 * cp;         // first column of the pair
    if (rb >= R || c >= C) return;
    uint32_t a[8], b[8];                   // bf16 pairs along R: column c, column c + 1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t w0 = tile[qc_word(16 * blk + 2 * i, cp)];
        const uint32_t w1 = tile[qc_word(16 * blk + 2 * i + 1, cp)];
        a[i] = (w0 & 0xFFFFu) | (w1 << 16);
        b[i] = (w0 >> 16) | (w1 & 0xFFFF0000u);
    }
    const int64_t half = R / 2, nb = R / 16;
    uint2 codes;
    uint32_t s8 = encode_block(a, Sg, t, codes);
    *reinterpret_cast<uint2*>(codes_t + c * half + rb / 2) = codes;
    scales_t[c * nb + rb / 16] = (uint8_t)s8;
    if (c + 1 < C) {
        s8 = encode_block(b, Sg, t, codes);
        *reinterpret_cast<uint2*>(codes_t + (c + 1) * half + rb / 2) = codes;
        scales_t[(c + 1) * nb + rb / 16] = (uint8_t)s8;
    }
}

// --------------------------------------------------- dequantize transpose --
// Tile: 128 rows x 128 columns of the rowwise tensor (-> 128 x 128 of y^T).
// Decode: thread t owns the row pair 2 (t / 4), +1 and the 32-column quarter
// t % 4 (16 code bytes of each row, so a load instruction of a wave covers 16
// rows x 64 bytes); it decodes both rows' two blocks and writes 32 words (one
// output row each: the two rows' values at one column) into the transposed
// LDS tile.  Word w of output row c sits at w ^ (16 * (c / 32)), which puts
// the 64 lanes of a wave's LDS writes on 64 different banks.  Store: 16 bytes
// (8 values) per thread, 16 threads per 256-byte output row.
constexpr int kDR = 128, kDC = 128;
constexpr int kDStride = kDR / 2 + 1;  // words per LDS row of y^T

__device__ __forceinline__ void dequant16(uint2 c, float s, float Sg, uint32_t out[8]) {
    const uint32_t cw[2] = {c.x, c.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        f32x2 q[4];
        fp4x8_to_f32(cw[h], q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float qs0 = q[i].x * s, qs1 = q[i].y * s;
            const float v0 = qs0 * Sg, v1 = qs1 * Sg;
            out[h * 4 + i] = f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16);
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_dequant_t(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        const float* __restrict__ sg_ptr, int64_t R,
                                                        int64_t C, uint16_t* __restrict__ y_t) {
    __shared__ uint32_t tile[kDC * kDStride];
    const float Sg = *sg_ptr;
    // blockIdx.x walks the row tiles, so workgroups that run together write
    // adjacent 256-byte pieces of the same output rows
    const int64_t r0 = (int64_t)blockIdx.x * kDR, c0 = (int64_t)blockIdx.y * kDC;
    const int p = threadIdx.x >> 2, q = threadIdx.x & 3;
    const int64_t r = r0 + 2 * p, cq = c0 + 32 * q;
    const int64_t bpr = C / 16;
    uint32_t v[2][2][8];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 8; ++i) v[a][b][i] = 0;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int64_t row = r + a;
        if (row >= R) continue;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int64_t c = cq + 16 * b;   // C % 16 == 0: a block is whole or absent
            if (c + 16 > C) continue;
            dequant16(*reinterpret_cast<const uint2*>(codes + row * (C / 2) + c / 2),
                      e4m3_to_f32(scales[row * bpr + c / 16]), Sg, v[a][b]);
        }
    }
    const int swz = q << 4;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int col = 32 * q + 16 * b + 2 * i;
            tile[col * kDStride + (p ^ swz)] = (v[0][b][i] & 0xFFFFu) | (v[1][b][i] << 16);
            tile[(col + 1) * kDStride + (p ^ swz)] = (v[0][b][i] >> 16) | (v[1][b][i] & 0xFFFF0000u);
        }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < kDC / 16; ++pass) {
        const int lrow = pass * 16 + (threadIdx.x >> 4), lw = (threadIdx.x & 15) * 4;
        const int64_t orow = c0 + lrow, ocol = r0 + 2 * lw;   // y^T [C, R]
        if (orow >= C || ocol >= R) continue;                // R % 8 == 0: whole 8-value pieces
        const uint32_t* src = tile + lrow * kDStride + (lw ^ ((lrow >> 5) << 4));
        const u32x4 w = {src[0], src[1], src[2], src[3]};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(y_t + orow * R + ocol));
    }
}

}  // namespace

hipError_t launch_quantize_cols(const uint16_t* x, int64_t rows, int64_t cols, ScaleMode mode,
                                const uint32_t* partial, int npartial, const float* sg_ptr, uint8_t* codes_t,
                                uint8_t* scales_t, float* global_out, hipStream_t stream) {
    const dim3 grid((unsigned)((cols + kQC - 1) / kQC), (unsigned)((rows + kQR - 1) / kQR));
    if (mode == ScaleMode::kDynamic)
        hipLaunchKernelGGL(k_quantize_cols<ScaleMode::kDynamic>, grid, dim3(kThreads), 0, stream, x, rows, cols,
                           partial, npartial, sg_ptr, codes_t, scales_t, global_out);
    else
        hipLaunchKernelGGL(k_quantize_cols<ScaleMode::kStatic>, grid, dim3(kThreads), 0, stream, x, rows, cols,
                           partial, npartial, sg_ptr, codes_t, scales_t, global_out);
    return hipGetLastError();
}

hipError_t launch_dequantize_t(const uint8_t* codes, const uint8_t* scales, const float* sg_ptr, int64_t rows,
                               int64_t cols, uint16_t* y_t, hipStream_t stream) {
    const dim3 grid((unsigned)((rows + kDR - 1) / kDR), (unsigned)((cols + kDC - 1) / kDC));
    hipLaunchKernelGGL(k_dequant_t, grid, dim3(kThreads), 0, stream, codes, scales, sg_ptr, rows, cols, y_t);
    return hipGetLastError();
}

}  // namespace nvfp4
