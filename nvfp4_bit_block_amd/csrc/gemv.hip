// gemv.hip -- batch 1..8 W4A16 GEMV on NVFP4 weights for gfx950.
//
// The decode-time projection the "vroomfondel/glm-5.2-reap-504B-v2-W4A4"
// model card targets ("What this variant changes": batch-1 decode GEMVs are
// pure weight bandwidth): y[m, n] = Sg * sum_b s[n, b] * sum_{k in b} q[n, k] x[m, k].
//
// One wavefront owns one output row at a time.  Each lane streams 16-byte
// chunks of packed codes (32 elements = two 16-element blocks) with the two
// matching scale bytes, decodes the codes to exact bf16 grid values with the
// gfx950 FP4 -> bf16 conversion, forms per-block partial dot products with
// v_dot2_f32_bf16 (fp32 accumulation), applies the block scale once per
// block, and the row sum is reduced across the wave at the end.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float dot2(bf16x2 a, uint32_t b_bits, float c) {
    bf16x2 b = __builtin_bit_cast(bf16x2, b_bits);
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

template <int M>
__global__ __launch_bounds__(kThreads) void k_gemv(const uint16_t* __restrict__ x, int64_t N,
                                                   int64_t K, const uint8_t* __restrict__ wc,
                                                   const uint8_t* __restrict__ ws,
                                                   const float* __restrict__ g0,
                                                   const float* __restrict__ g1,
                                                   uint16_t* __restrict__ y) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);
    const float scale = *g0 * (g1 ? *g1 : 1.0f);
    const int64_t nchunk = K / 32;
    for (int64_t n = (int64_t)blockIdx.x * (kThreads / kWave) + (threadIdx.x / kWave); n < N;
         n += nwaves) {
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;
        const uint4* wrow = reinterpret_cast<const uint4*>(wc + n * (K / 2));
        const uint16_t* srow = reinterpret_cast<const uint16_t*>(ws + n * (K / 16));
#pragma unroll 2
        for (int64_t c = lane; c < nchunk; c += kWave) {
            const uint4 q = load_nt16(&wrow[c]);
            const uint32_t s2 = __builtin_nontemporal_load(&srow[c]);
            const float s0 = e4m3_to_f32(s2 & 0xFFu);
            const float s1 = e4m3_to_f32(s2 >> 8);
            bf16x2 wv[16];
            fp4x8_to_bf16(q.x, &wv[0]);
            fp4x8_to_bf16(q.y, &wv[4]);
            fp4x8_to_bf16(q.z, &wv[8]);
            fp4x8_to_bf16(q.w, &wv[12]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint4* xr = reinterpret_cast<const uint4*>(x + m * K + c * 32);
                const uint4 xa = xr[0], xb = xr[1], xc = xr[2], xd = xr[3];
                float p0 = 0.0f, p1 = 0.0f;
                p0 = dot2(wv[0], xa.x, p0);
                p0 = dot2(wv[1], xa.y, p0);
                p0 = dot2(wv[2], xa.z, p0);
                p0 = dot2(wv[3], xa.w, p0);
                p0 = dot2(wv[4], xb.x, p0);
                p0 = dot2(wv[5], xb.y, p0);
                p0 = dot2(wv[6], xb.z, p0);
                p0 = dot2(wv[7], xb.w, p0);
                p1 = dot2(wv[8], xc.x, p1);
                p1 = dot2(wv[9], xc.y, p1);
                p1 = dot2(wv[10], xc.z, p1);
                p1 = dot2(wv[11], xc.w, p1);
                p1 = dot2(wv[12], xd.x, p1);
                p1 = dot2(wv[13], xd.y, p1);
                p1 = dot2(wv[14], xd.z, p1);
                p1 = dot2(wv[15], xd.w, p1);
                acc[m] = __builtin_fmaf(s0, p0, acc[m]);
                acc[m] = __builtin_fmaf(s1, p1, acc[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = wave_sum(acc[m]);
        if (lane == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) y[m * N + n] = (uint16_t)f32_to_bf16_rne(acc[m] * scale);
        }
    }
}

template <int M>
hipError_t launch_m(const uint16_t* x, int64_t N, int64_t K, const uint8_t* wc, const uint8_t* ws,
                    const float* g0, const float* g1, uint16_t* y, hipStream_t stream) {
    const int64_t waves_per_block = kThreads / kWave;
    int64_t grid = (N + waves_per_block - 1) / waves_per_block;
    if (grid > 65535) grid = 65535;
    hipLaunchKernelGGL(k_gemv<M>, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, N, K, wc, ws,
                       g0, g1, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_w4a16(const uint16_t* x, int M, int64_t N, int64_t K, const uint8_t* wc,
                             const uint8_t* ws, const float* g0, const float* g1, uint16_t* y,
                             hipStream_t stream) {
    switch (M) {
        case 1: return launch_m<1>(x, N, K, wc, ws, g0, g1, y, stream);
        case 2: return launch_m<2>(x, N, K, wc, ws, g0, g1, y, stream);
        case 3: return launch_m<3>(x, N, K, wc, ws, g0, g1, y, stream);
        case 4: return launch_m<4>(x, N, K, wc, ws, g0, g1, y, stream);
        case 5: return launch_m<5>(x, N, K, wc, ws, g0, g1, y, stream);
        case 6: return launch_m<6>(x, N, K, wc, ws, g0, g1, y, stream);
        case 7: return launch_m<7>(x, N, K, wc, ws, g0, g1, y, stream);
        case 8: return launch_m<8>(x, N, K, wc, ws, g0, g1, y, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4
