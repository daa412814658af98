// gemv.hip -- batch 1..8 W4A16 GEMV on NVFP4 weights for gfx950.
//
// The decode-time projection the "vroomfondel/glm-5.2-reap-504B-v2-W4A4"
// model card targets ("What this variant changes": batch-1 decode GEMVs are
// pure weight bandwidth): y[m, n] = Sg * sum_b s[n, b] * sum_{k in b} q[n, k] x[m, k].
//
// The kernel is HBM-bound: it must keep enough weight bytes in flight and
// spend only ~1-2 VALU lane-ops per weight element.  Layout of the work:
//   * a wavefront owns RW output rows at a time; lane l owns the 32-element
//     chunks c = l + 64 j (j < NCH) of each row, so every 16-byte load
//     instruction of the wave reads 1 KB of contiguous packed codes;
//   * all NCH chunk loads (and their 2 scale bytes) of the RW rows are issued
//     before any is used, so a wave has RW*NCH KB in flight;
//   * codes are decoded to exact bf16 grid values by the gfx950 FP4 -> bf16
//     conversion (one instruction per two elements) and multiplied with the
//     activation by v_dot2_f32_bf16, one fp32 partial per 16-element block,
//     scaled once per block;
//   * the activation is read once per workgroup: k_gemv (the fixed layouts,
//     K = 2048 times 1, 2, 4, 8 or 16) holds each lane's slice of it in VGPRs
//     for every M <= 8; k_gemv_any (other K) stages it in LDS when
//     M * K * 2 <= 64 KB and reads it from global memory otherwise;
//   * row sums are reduced across the wave with cross-lane shuffles.
// Weights are read with non-temporal loads: each byte is used once.
#include "nvfp4_device.hpp"
#include "nvfp4_encode.hpp"
#include "nvfp4_internal.hpp"

#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float dot2(bf16x2 a, uint32_t b_bits, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b_bits), c, false);
}

// Partial dot products of one 32-element chunk (two blocks) with M activation
// rows; x4(m, i) returns the i-th 16-byte piece (8 bf16) of row m's chunk.
template <int M, typename XF>
__device__ __forceinline__ void chunk_dot(uint4 q, uint32_t s2, XF x4, float acc[M]) {
    const f32x2 sc = e4m3x2_to_f32(s2);
    const float s0 = sc.x, s1 = sc.y;
    bf16x2 wv[16];
    fp4x8_to_bf16(q.x, &wv[0]);
    fp4x8_to_bf16(q.y, &wv[4]);
    fp4x8_to_bf16(q.z, &wv[8]);
    fp4x8_to_bf16(q.w, &wv[12]);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint4 xa = x4(m, 0), xb = x4(m, 1), xc = x4(m, 2), xd = x4(m, 3);
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

// Activation in LDS, transposed so that lanes reading the same 16-byte piece
// of consecutive chunks hit consecutive LDS addresses (no bank conflicts):
// piece p (8 bf16) of chunk c of row m lives at [(m * 4 + p) * nchunk + c].
template <int M, int THREADS>
__device__ __forceinline__ void stage_x_lds(uint4* xlds, const uint16_t* __restrict__ x, int64_t K) {
    const uint4* src = reinterpret_cast<const uint4*>(x);
    const int64_t per_row = K / 8, nchunk = K / 32;
    for (int64_t g = threadIdx.x; g < (int64_t)M * per_row; g += THREADS) {
        const int64_t m = g / per_row, r = g - m * per_row;
        xlds[(m * 4 + (r & 3)) * nchunk + (r >> 2)] = src[g];
    }
    __syncthreads();
}

// Weight fragment: for RW rows, NCH 16-byte code chunks and their two scale
// bytes per lane.
template <int RW, int NCH>
struct Frag {
    uint4 q[RW][NCH];
    uint32_t s[RW][NCH];
};

// Fixed chunk layout: K == KS * NCH * 2048.  A workgroup of THREADS / 64
// waves forms row groups of KS waves; the KS waves of a group split K (wave part p
// owns chunks p*64*NCH + lane + 64*j, j < NCH), so each lane keeps only its
// NCH chunks of the activation in VGPRs.  A row group walks its batches of RW
// rows with one fragment of registers: the registers of chunk j are refilled
// with the next batch's chunk j right after use, so a whole fragment of loads
// is in flight while the wave computes.  The last batch is peeled so the
// refill is unconditional (no register copies).  Partial row sums are reduced
// across the wave with shuffles and, when KS > 1, across the group's waves
// through LDS.
//
// With AP (the W4A4 product on a pre-packed activation) x points to the
// activation's packed codes [M, K/2] and xs to its E4M3 scales [M, K/16]: each
// lane decodes its slice to the exact products q * s as bf16 (the values the
// expanded operand would hold), and g1 is the activation's global scale.
//
// With AQ (the W4A4 product at M = 1) x is the unquantized bf16 activation:
// each lane NVFP4-encodes its slice under the static activation scale *g1
// (the quantizer's block rule) and keeps the exact products q * s as bf16,
// the operand the two-kernel path would read back from memory.
template <int M, int NCH, int KS, int RW, int THREADS = kThreads, bool AQ = false, bool AP = false>
__global__ __launch_bounds__(THREADS) void k_gemv(const uint16_t* __restrict__ x, int64_t N,
                                                   int64_t K, const uint8_t* __restrict__ wc,
                                                   const uint8_t* __restrict__ ws,
                                                   const float* __restrict__ g0,
                                                   const float* __restrict__ g1,
                                                   uint16_t* __restrict__ y,
                                                   const uint8_t* __restrict__ xs) {
    constexpr int kWavesPerBlock = THREADS / kWave;
    constexpr int kGroups = kWavesPerBlock / KS;
    static_assert(kWavesPerBlock % KS == 0, "row groups");
    __shared__ float red[2][kWavesPerBlock][RW][M];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int grp = wave / KS, part = wave % KS;
    const int64_t KB = K / 2, KS16 = K / 16;
    // chunk of (lane, j): lane + 64 j of the part, so every load instruction
    // of the wave reads 1 KB contiguous
    const int64_t cbase = (int64_t)part * 64 * NCH;
    auto chunk = [&](int j) -> int64_t { return cbase + lane + 64 * j; };

    // batches of RW rows: this group owns b = gid, gid + ngroups, ...
    const int64_t nbatch = (N + RW - 1) / RW;
    const int64_t gid = (int64_t)blockIdx.x * kGroups + grp;
    const int64_t ngroups = (int64_t)gridDim.x * kGroups;
    // every wave of a workgroup runs the same number of iterations (the LDS
    // reduction synchronizes them); batches past the end are computed on a
    // clamped row and not stored
    const int64_t iters = (nbatch + ngroups - 1) / ngroups;
    const int64_t my_iters = (KS > 1) ? iters : (gid < nbatch ? (nbatch - 1 - gid) / ngroups + 1 : 0);

    // one row's chunks and scale pairs into fragment slot r
    auto load_row = [&](Frag<RW, NCH>& f, int r, const uint8_t* wrow, const uint16_t* srow) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            f.q[r][j] = load_nt16(wrow + chunk(j) * 16);
            f.s[r][j] = __builtin_nontemporal_load(srow + chunk(j));
        }
    };

    auto load = [&](Frag<RW, NCH>& f, int64_t b) {
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int64_t row = min(b * RW + r, N - 1);
            const uint8_t* wrow = wc + row * KB;
            const uint16_t* srow = reinterpret_cast<const uint16_t*>(ws + row * KS16);
            load_row(f, r, wrow, srow);
        }
    };

    // Load order: with several batch rows the activation's loads go first,
    // so that the first products (and the AP decode or AQ encode) wait for
    // them alone while the first weight batch is in flight (waits on loads
    // are in issue order); measured on MI355X, o_proj M = 2 / 4 13.9 / 19.3
    // -> 13.4 / 18.8 us, q_b_proj M = 2 7.00 -> 6.71 us.  At M = 1 the
    // weights go first (the other order measured 0.4-1.3 % slower).
    uint4 xr[M * NCH * 4];
    uint4 xq[AP ? M * NCH : 1];
    uint32_t xs2[AP ? M * NCH : 1];
    auto load_x = [&]() {
        if constexpr (AP) {
            // chunk c of row m: 16 code bytes (two blocks) and their two scale bytes
            const uint8_t* xc = reinterpret_cast<const uint8_t*>(x);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    xq[m * NCH + j] = *reinterpret_cast<const uint4*>(xc + m * KB + chunk(j) * 16);
                    xs2[m * NCH + j] = *reinterpret_cast<const uint16_t*>(xs + m * KS16 + chunk(j) * 2);
                }
        } else {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const uint4* p = reinterpret_cast<const uint4*>(x + m * K + chunk(j) * 32);
#pragma unroll
                    for (int i = 0; i < 4; ++i) xr[(m * NCH + j) * 4 + i] = p[i];
                }
        }
    };
    Frag<RW, NCH> f;
    if constexpr (M > 1) load_x();
    if (my_iters > 0) load(f, gid);
    if constexpr (M == 1) load_x();

    if constexpr (AP) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint4 q = xq[m * NCH + j];
                const uint32_t s2 = xs2[m * NCH + j];
                const float s0 = e4m3_to_f32(s2 & 0xFFu), s1 = e4m3_to_f32(s2 >> 8);
                uint4* o = &xr[(m * NCH + j) * 4];
                o[0] = fp4x8_scaled_bf16_bits(q.x, s0);
                o[1] = fp4x8_scaled_bf16_bits(q.y, s0);
                o[2] = fp4x8_scaled_bf16_bits(q.z, s1);
                o[3] = fp4x8_scaled_bf16_bits(q.w, s1);
            }
    }
    if constexpr (AQ) {
        const float sg = *g1, t = 6.0f * sg;
#pragma unroll
        for (int p = 0; p < M * NCH * 2; ++p) {
            // 16-element block p: pieces 2p, 2p + 1 of the lane's slice
            uint4& a = xr[2 * p];
            uint4& b = xr[2 * p + 1];
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint2 codes;
            const float sc = e4m3_to_f32(encode_block(w, sg, t, codes));
            a = fp4x8_scaled_bf16_bits(codes.x, sc);
            b = fp4x8_scaled_bf16_bits(codes.y, sc);
        }
    }
    const float scale = *g0 * (g1 ? *g1 : 1.0f);

    auto finish = [&](float (&acc)[RW][M], int64_t b, int it) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = wave_sum_lane63(acc[r][m]);
        if constexpr (KS == 1) {
            if (lane == kWave - 1 && b < nbatch) {
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    if (b * RW + r >= N) break;
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        y[m * N + b * RW + r] = (uint16_t)f32_to_bf16_rne(acc[r][m] * scale);
                }
            }
        } else {
            const int buf = it & 1;
            if (lane == kWave - 1) {
#pragma unroll
                for (int r = 0; r < RW; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m) red[buf][wave][r][m] = acc[r][m];
            }
            __syncthreads();
            if (part == 0 && lane < RW * M && b < nbatch) {
                const int r = lane / M, m = lane % M;
                float v = 0.0f;
#pragma unroll
                for (int p = 0; p < KS; ++p) v += red[buf][grp * KS + p][r][m];
                if (b * RW + r < N) y[m * N + b * RW + r] = (uint16_t)f32_to_bf16_rne(v * scale);
            }
        }
    };

    // compute the batch held in f; with PREFETCH, refill f with batch bn
    auto compute = [&](auto prefetch, float (&acc)[RW][M], int64_t bn) {
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int64_t row = min(bn * RW + r, N - 1);
            const uint8_t* wrow = wc + row * KB;
            const uint16_t* srow = reinterpret_cast<const uint16_t*>(ws + row * KS16);
#pragma unroll
            for (int j = 0; j < NCH; ++j)
                chunk_dot<M>(f.q[r][j], f.s[r][j],
                             [&](int m, int i) { return xr[(m * NCH + j) * 4 + i]; }, acc[r]);
            if constexpr (decltype(prefetch)::value) load_row(f, r, wrow, srow);
        }
    };

    int64_t b = gid;
    for (int64_t it = 0; it + 1 < my_iters; ++it, b += ngroups) {
        float acc[RW][M] = {};
        compute(std::true_type{}, acc, b + ngroups);
        finish(acc, b, (int)it);
    }
    if (my_iters > 0) {
        float acc[RW][M] = {};
        compute(std::false_type{}, acc, 0);
        finish(acc, b, (int)(my_iters - 1));
    }
}

// Any K % 32 == 0: chunk loop at run time, four chunks in flight per lane;
// activation from LDS when it fits, else from global memory.
template <int M, bool XLDS, int THREADS>
__global__ __launch_bounds__(THREADS) void k_gemv_any(const uint16_t* __restrict__ x, int64_t N,
                                                      int64_t K, const uint8_t* __restrict__ wc,
                                                      const uint8_t* __restrict__ ws,
                                                      const float* __restrict__ g0,
                                                      const float* __restrict__ g1,
                                                      uint16_t* __restrict__ y) {
    extern __shared__ uint4 xlds[];
    constexpr int kWavesPerBlock = THREADS / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const float scale = *g0 * (g1 ? *g1 : 1.0f);
    const int64_t nchunk = K / 32;
    const int64_t KB = K / 2, KS = K / 16;
    if constexpr (XLDS) stage_x_lds<M, THREADS>(xlds, x, K);
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t n = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave); n < N; n += nwaves) {
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;
        const uint8_t* wrow = wc + n * KB;
        const uint16_t* srow = reinterpret_cast<const uint16_t*>(ws + n * KS);
        for (int64_t c0 = lane; c0 < nchunk; c0 += 4 * kWave) {
            uint4 q[4];
            uint32_t s[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t c = min(c0 + u * kWave, nchunk - 1);
                q[u] = load_nt16(wrow + c * 16);
                s[u] = __builtin_nontemporal_load(srow + c);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t c = c0 + u * kWave;
                if (c < nchunk) {
                    chunk_dot<M>(q[u], s[u],
                                 [&](int m, int i) {
                                     if constexpr (XLDS) return xlds[(m * 4 + i) * nchunk + c];
                                     else return reinterpret_cast<const uint4*>(x + m * K + c * 32)[i];
                                 },
                                 acc);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = wave_sum_lane63(acc[m]);
        if (lane == kWave - 1) {
#pragma unroll
            for (int m = 0; m < M; ++m) y[m * N + n] = (uint16_t)f32_to_bf16_rne(acc[m] * scale);
        }
    }
}

constexpr int64_t kMaxLdsBytes = 64 * 1024;

// Grid: about `blocks_per_cu` workgroups per CU on a 256-CU chip, never
// more than there are row batches.
template <int M, int NCH, int KS, int RW, int THREADS = kThreads, bool AQ = false, bool AP = false>
hipError_t launch_cfg(const uint16_t* x, int64_t N, int64_t K, const uint8_t* wc, const uint8_t* ws,
                      const float* g0, const float* g1, uint16_t* y, hipStream_t stream,
                      int blocks_per_cu, const uint8_t* xs = nullptr) {
    constexpr int64_t groups = (THREADS / kWave) / KS;
    const int64_t nbatch = (N + RW - 1) / RW;
    int64_t grid = min((int64_t)256 * blocks_per_cu, (nbatch + groups - 1) / groups);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((k_gemv<M, NCH, KS, RW, THREADS, AQ, AP>), dim3((unsigned)grid), dim3(THREADS), 0, stream, x,
                       N, K, wc, ws, g0, g1, y, xs);
    return hipGetLastError();
}

template <int M, bool XLDS>
hipError_t launch_any(const uint16_t* x, int64_t N, int64_t K, const uint8_t* wc, const uint8_t* ws,
                      const float* g0, const float* g1, uint16_t* y, hipStream_t stream) {
    int64_t grid = (N + 3) / 4;
    if (grid > 2048) grid = 2048;
    const size_t lds = XLDS ? (size_t)M * (size_t)K * 2 : 0;
    hipLaunchKernelGGL((k_gemv_any<M, XLDS, kThreads>), dim3((unsigned)grid), dim3(kThreads), lds, stream,
                       x, N, K, wc, ws, g0, g1, y);
    return hipGetLastError();
}

template <int M, bool AQ = false, bool AP = false>
hipError_t launch_m(const uint16_t* x, int64_t N, int64_t K, const uint8_t* wc, const uint8_t* ws,
                    const float* g0, const float* g1, uint16_t* y, hipStream_t stream,
                    const uint8_t* xs = nullptr) {
    const bool fits_lds = (int64_t)M * K * 2 <= kMaxLdsBytes;
    // K = 2048 KS: KS waves split a row, each lane owning one 32-element
    // chunk per batch row, four rows in flight per wave.  Measured on MI355X
    // (o_proj 6144 x 16384 and q_b_proj 16384 x 2048): K = 2048, one wave per
    // row, three workgroups per CU (two for M > 4); K = 16384, eight waves
    // per row in one 512-thread workgroup per CU.  The other multiples take
    // the nearest of these arrangements.
    if (K % 2048 == 0) {
        switch (K / 2048) {
            case 1: return launch_cfg<M, 1, 1, 4, kThreads, AQ, AP>(x, N, K, wc, ws, g0, g1, y, stream, M <= 4 ? 3 : 2, xs);
            case 2: return launch_cfg<M, 1, 2, 4, kThreads, AQ, AP>(x, N, K, wc, ws, g0, g1, y, stream, 2, xs);
            case 4: return launch_cfg<M, 1, 4, 4, 512, AQ, AP>(x, N, K, wc, ws, g0, g1, y, stream, 1, xs);
            case 8: return launch_cfg<M, 1, 8, 4, 512, AQ, AP>(x, N, K, wc, ws, g0, g1, y, stream, 1, xs);
            case 16: return launch_cfg<M, 1, 16, 4, 1024, AQ, AP>(x, N, K, wc, ws, g0, g1, y, stream, 1, xs);
            default: break;
        }
    }
    if constexpr (AQ || AP) return hipErrorNotSupported;
    if (fits_lds) return launch_any<M, true>(x, N, K, wc, ws, g0, g1, y, stream);
    return launch_any<M, false>(x, N, K, wc, ws, g0, g1, y, stream);
}

hipError_t launch_batch(const uint16_t* x, int M, int64_t N, int64_t K, const uint8_t* wc,
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

}  // namespace

hipError_t launch_gemv_w4a16(const uint16_t* x, int M, int64_t N, int64_t K, const uint8_t* wc,
                             const uint8_t* ws, const float* g0, const float* g1, uint16_t* y,
                             hipStream_t stream) {
    return launch_batch(x, M, N, K, wc, ws, g0, g1, y, stream);
}

// Measured on MI355X: the in-register quantize costs each lane 2 M block
// encodes up front; at M = 1 that hides behind the first weight loads and
// saves the separate quantize launch, from M = 2 on the two-kernel path is
// as fast or faster.
namespace {
// K of the fixed chunk layouts (2048 times 1, 2, 4, 8 or 16)
bool fixed_layout(int64_t K) {
    if (K % 2048 != 0) return false;
    const int64_t ks = K / 2048;
    return ks == 1 || ks == 2 || ks == 4 || ks == 8 || ks == 16;
}
}  // namespace

bool gemv_quantizes_activation(int M, int64_t K) { return M == 1 && fixed_layout(K); }

hipError_t launch_gemv_w4a4(const uint16_t* x, int M, int64_t N, int64_t K, const uint8_t* wc,
                            const uint8_t* ws, const float* w_global, const float* input_scale,
                            uint16_t* y, hipStream_t stream) {
    if (!gemv_quantizes_activation(M, K)) return hipErrorNotSupported;
    return launch_m<1, true>(x, N, K, wc, ws, w_global, input_scale, y, stream);
}

// The fixed chunk layouts (K = 2048 times 1, 2, 4, 8 or 16) decode a packed
// activation in registers; other K expand it to q * s in memory first.
bool gemv_takes_packed(int M, int64_t K) { return M >= 1 && M <= 8 && fixed_layout(K); }

hipError_t launch_gemv_w4a4_packed(const uint8_t* a_codes, const uint8_t* a_scales, int M, int64_t N, int64_t K,
                                   const uint8_t* wc, const uint8_t* ws, const float* w_global,
                                   const float* a_global, uint16_t* y, hipStream_t stream) {
    if (!gemv_takes_packed(M, K)) return hipErrorNotSupported;
    const uint16_t* xc = reinterpret_cast<const uint16_t*>(a_codes);
    switch (M) {
        case 1: return launch_m<1, false, true>(xc, N, K, wc, ws, w_global, a_global, y, stream, a_scales);
        case 2: return launch_m<2, false, true>(xc, N, K, wc, ws, w_global, a_global, y, stream, a_scales);
        case 3: return launch_m<3, false, true>(xc, N, K, wc, ws, w_global, a_global, y, stream, a_scales);
        case 4: return launch_m<4, false, true>(xc, N, K, wc, ws, w_global, a_global, y, stream, a_scales);
        case 5: return launch_m<5, false, true>(xc, N, K, wc, ws, w_global, a_global, y, stream, a_scales);
        case 6: return launch_m<6, false, true>(xc, N, K, wc, ws, w_global, a_global, y, stream, a_scales);
        case 7: return launch_m<7, false, true>(xc, N, K, wc, ws, w_global, a_global, y, stream, a_scales);
        case 8: return launch_m<8, false, true>(xc, N, K, wc, ws, w_global, a_global, y, stream, a_scales);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4
