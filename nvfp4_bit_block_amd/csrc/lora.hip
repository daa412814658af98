// lora.hip -- the rank-r projection through LoRA's shared A matrix, the first
// half of the non-fused MoE-LoRA path ("Getting GLM-5.2 NVFP4 Post-Training
// off the ground", "Going deeper": a rank-64 bf16 LoRA on the MLP of an NVFP4
// base, one LoRA-A shared by all routed experts, one LoRA-B per expert).
// Because A is shared, the projection is one dense product over all rows;
// the per-expert B half runs in the grouped GEMM epilogue.
//
//   Z [rows, R] = bf16(X [rows, K] * A [R, K]^T), fp32 accumulation.
//
// One workgroup owns 32 rows; its eight waves split K, each with two steps of
// loads in flight, and their fp32 partial blocks are summed in wave order
// through LDS.  Each wave multiplies on
// v_mfma_f32_32x32x16_bf16 with operands loaded straight from global memory:
// per 64-wide K step, lane (c, h) reads 64 contiguous bytes of row c of X and
// of row c of each 32-row block of A at K offset 32 h, and MFMA kk takes
// positions 32 h + 8 kk + [0, 8) -- the same K permutation on both operands,
// so the product is unchanged.  R is padded to 32-column blocks with zeros.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kWaves = 8;

template <int NCB>
__global__ __launch_bounds__(64 * kWaves) void k_lora_a(const uint16_t* __restrict__ x, int64_t rows,
                                                        int64_t K, const uint16_t* __restrict__ a, int R,
                                                        uint16_t* __restrict__ z) {
    __shared__ f32x16 red[kWaves - 1][NCB][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c32 = lane & 31, hf = lane >> 5;
    const int64_t rb = (int64_t)blockIdx.x * 32, row = rb + c32;
    const int ksteps = (int)(K / 64);
    const int per = (ksteps + kWaves - 1) / kWaves;
    const int s0 = min(ksteps, wave * per), s1 = min(ksteps, s0 + per);

    const uint16_t* xp = row < rows ? x + row * K + 32 * hf : nullptr;
    const uint16_t* ap[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = 32 * cb + c32;
        ap[cb] = col < R ? a + (int64_t)col * K + 32 * hf : nullptr;
    }
    struct Step {
        u32x4 x[4], a[NCB][4];
    };
    auto load = [&](int s, Step& st) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            st.x[u] = u32x4{0, 0, 0, 0};
            if (xp) st.x[u] = *reinterpret_cast<const u32x4*>(xp + 64 * (int64_t)s + 8 * u);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                st.a[cb][u] = u32x4{0, 0, 0, 0};
                if (ap[cb]) st.a[cb][u] = *reinterpret_cast<const u32x4*>(ap[cb] + 64 * (int64_t)s + 8 * u);
            }
    };
    f32x16 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.0f;
    auto compute = [&](const Step& st) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, st.x[kk]),
                                                                  __builtin_bit_cast(bf16x8, st.a[cb][kk]), acc[cb],
                                                                  0, 0, 0);
    };
    // two steps of loads in flight: even steps in p, odd steps in q
    Step p, q;
    if (s0 < s1) load(s0, p);
    if (s0 + 1 < s1) load(s0 + 1, q);
    for (int s = s0; s < s1; s += 2) {
        compute(p);
        if (s + 2 < s1) load(s + 2, p);
        if (s + 1 < s1) {
            compute(q);
            if (s + 3 < s1) load(s + 3, q);
        }
    }

    if (wave > 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) red[wave - 1][cb][lane] = acc[cb];
    }
    __syncthreads();
    if (wave != 0) return;
    // lane holds rows 8 (r/4) + 4 hf + r%4 of the block, column c32 of each column block
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        f32x16 v = acc[cb];
#pragma unroll
        for (int w = 0; w < kWaves - 1; ++w) v += red[w][cb][lane];
        const int col = 32 * cb + c32;
        if (col >= R) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t orow = rb + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (orow < rows) z[orow * R + col] = (uint16_t)f32_to_bf16_rne(v[r]);
        }
    }
}

}  // namespace

hipError_t launch_lora_a(const uint16_t* x, int64_t rows, int64_t K, const uint16_t* a, int R, uint16_t* z,
                         hipStream_t stream) {
    const dim3 grid((unsigned)((rows + 31) / 32)), block(64 * kWaves);
    switch ((R + 31) / 32) {
        case 1: hipLaunchKernelGGL(k_lora_a<1>, grid, block, 0, stream, x, rows, K, a, R, z); break;
        case 2: hipLaunchKernelGGL(k_lora_a<2>, grid, block, 0, stream, x, rows, K, a, R, z); break;
        case 3: hipLaunchKernelGGL(k_lora_a<3>, grid, block, 0, stream, x, rows, K, a, R, z); break;
        case 4: hipLaunchKernelGGL(k_lora_a<4>, grid, block, 0, stream, x, rows, K, a, R, z); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace nvfp4
