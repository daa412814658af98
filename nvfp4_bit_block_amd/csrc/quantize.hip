// quantize.hip -- NVFP4 quantize (two-pass dynamic, one-pass static) and
// dequantize for gfx950.
//
// Format and scale rule: "vroomfondel/glm-5.2-reap-504B-v2-W4A4" model card,
// "How it was produced" (e2m1 codes, per-16 e4m3 block scales stored
// linearly, per-tensor fp32 scale amax / (6 * 448); static input_scale for
// activations); "Getting GLM-5.2 NVFP4 Post-Training off the ground",
// "Going deeper" (16-element blocks along the row, two codes per byte) and
// "The bottom line" (a block's scale follows the block maximum).
//
// Every decision is taken with the same fp32 operations as the definition:
// Sg = amax / 2688, t = 6 * Sg, s_f = bmax / t, s8 = E4M3(s_f), d = s * Sg,
// v = |x| / d, code = sign | E2M1(v), each quotient correctly rounded (the
// build uses correctly rounded fp32 division and keeps denormals; the
// per-element quotients use an exact reciprocal-and-correct sequence).
#include "nvfp4_device.hpp"
#include "nvfp4_encode.hpp"
#include "nvfp4_internal.hpp"

#include <mutex>

// Bit-exactness needs every fp32 step rounded on its own: no contraction.
#pragma clang fp contract(off)

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
// static quantizes of at most this many blocks run four lanes per block
constexpr int64_t kQuadMaxBlocks = (int64_t)1 << 20;

// Pass 1: per-workgroup maximum of |x| as a bf16 magnitude pattern (for finite
// values the pattern order is the value order).  Grid-stride over 16-byte
// chunks of 8 elements with kAmaxUnroll independent loads in flight per
// thread (measured on MI355X over 65536 x 6144: 512-thread workgroups with
// eight loads each read at 7.0 TB/s on the grid below, 256 threads with four
// at 5.6 TB/s).
constexpr int kAmaxThreads = 512;
constexpr int kAmaxUnroll = 8;

__global__ __launch_bounds__(kAmaxThreads) void k_amax_partial(const uint4* __restrict__ x, int64_t n8,
                                                               uint32_t* __restrict__ partial) {
    uint32_t m0 = 0, m1 = 0;
    const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
    int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
    for (; i + (kAmaxUnroll - 1) * stride < n8; i += kAmaxUnroll * stride) {
        uint4 v[kAmaxUnroll];
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) v[u] = load_nt16(&x[i + u * stride]);
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) {
            uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t a = w[j] & 0x7FFF7FFFu;
                m0 = max(m0, a & 0xFFFFu);
                m1 = max(m1, a >> 16);
            }
        }
    }
    for (; i < n8; i += stride) {
        uint4 v = load_nt16(&x[i]);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t a = w[j] & 0x7FFF7FFFu;
            m0 = max(m0, a & 0xFFFFu);
            m1 = max(m1, a >> 16);
        }
    }
    uint32_t m = wave_max_u32(max(m0, m1));
    __shared__ uint32_t red[kAmaxThreads / kWave];
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
#pragma unroll
        for (int w = 1; w < kAmaxThreads / kWave; ++w) r = max(r, red[w]);
        partial[blockIdx.x] = r;
    }
}

// Pass 2 (or the only pass in the static modes): one 16-element block per
// thread per iteration, grid-stride.  The dynamic mode first reduces the
// pass-1 maxima (every workgroup does so redundantly; there are at most 2048).
template <ScaleMode MODE>
__global__ __launch_bounds__(kThreads) void k_quantize_pack(PackArgs a) {
    float Sg = 0.0f;
    if constexpr (MODE == ScaleMode::kDynamic) {
        uint32_t m = 0;
        for (int i = threadIdx.x; i < a.npartial; i += kThreads) m = max(m, a.partial[i]);
        m = wave_max_u32(m);
        __shared__ uint32_t red[kThreads / kWave];
        if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
        __syncthreads();
        m = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) m = max(m, red[w]);
        Sg = bf16_to_f32(m) / 2688.0f;
    } else if constexpr (MODE == ScaleMode::kStatic) {
        Sg = *a.sg_ptr;
    }
    if constexpr (MODE != ScaleMode::kGrouped) {
        if (a.global_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *a.global_out = Sg;
    }
    // Grouped scales that are all one value: quantize the ungathered source
    // rows once each (see PackArgs::n_groups).
    bool shared = false;
    if constexpr (MODE == ScaleMode::kGrouped) {
        if (a.n_groups > 0) {
            const uint32_t s0 = __float_as_uint(a.sg_group[0]);
            bool eq = true;
            for (int e = threadIdx.x; e < a.n_groups; e += kThreads) eq = eq && __float_as_uint(a.sg_group[e]) == s0;
            shared = __syncthreads_and(eq ? 1 : 0) != 0;
            if (blockIdx.x == 0 && threadIdx.x == 0) *a.shared_out = shared ? 1 : 0;
            if (shared) Sg = a.sg_group[0];
        }
    }
    float t = 6.0f * Sg;
    const int64_t bpr = a.cols / 16;
    const int64_t rows_valid =
        shared ? min(a.shared_rows, a.rows) : (a.rows_valid ? (int64_t)*a.rows_valid : a.rows);
    // blocks of the valid rows
    const int64_t nblk = min(a.rows, max(rows_valid, (int64_t)0)) * bpr;
    // Two blocks per thread per iteration (b and b + stride), both loads issued
    // before either block is encoded.  A slot past the end loads block 0 of
    // source row 0 instead and stores nothing; rows at or beyond rows_valid
    // (whose gather index may be unset) are never visited.
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t b0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; b0 < nblk; b0 += 2 * stride) {
        uint4 v[2][2];
        int64_t rr[2], cbb[2];
        bool ok[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int64_t b = b0 + p * stride;
            const int64_t r = (b < nblk ? b : b0) / bpr;
            ok[p] = b < nblk;
            rr[p] = r;
            cbb[p] = (b < nblk ? b : b0) - r * bpr;
            const int64_t sr = !ok[p] ? 0 : (!shared && a.src_row ? (int64_t)(a.src_row[r] / a.src_div) : r);
            const uint4* src = reinterpret_cast<const uint4*>(a.x + sr * a.cols + (ok[p] ? cbb[p] * 16 : 0));
            v[p][0] = load_nt16(src);
            v[p][1] = load_nt16(src + 1);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (!ok[p]) continue;
            const int64_t b = b0 + p * stride, r = rr[p], cb = cbb[p];
            if constexpr (MODE == ScaleMode::kGrouped) {
                if (!shared) {
                    Sg = a.sg_group[a.row_group[r]];
                    t = 6.0f * Sg;
                }
            }
            uint32_t w[8] = {v[p][0].x, v[p][0].y, v[p][0].z, v[p][0].w,
                             v[p][1].x, v[p][1].y, v[p][1].z, v[p][1].w};
            uint2 codes;
            uint32_t s8 = encode_block(w, Sg, t, codes);
            if (a.codes != nullptr) {
                reinterpret_cast<uint2*>(a.codes)[b] = codes;
                a.scales[b] = (uint8_t)s8;
            }
            if (a.xhat != nullptr) {
                // q * s for the 16 elements, exact in f16 and bf16
                const float s = e4m3_to_f32(s8);
                uint4* dst = reinterpret_cast<uint4*>(a.xhat + r * a.cols + cb * 16);
                if (a.xhat_bf16) {
                    dst[0] = fp4x8_scaled_bf16_bits(codes.x, s);
                    dst[1] = fp4x8_scaled_bf16_bits(codes.y, s);
                } else {
                    dst[0] = __builtin_bit_cast(uint4, fp4x8_scaled_f16(codes.x, (_Float16)s));
                    dst[1] = __builtin_bit_cast(uint4, fp4x8_scaled_f16(codes.y, (_Float16)s));
                }
            }
        }
    }
}

// Small static-scale inputs without a gather: four lanes per 16-element
// block, each holding four consecutive elements (one 8-byte load, so a wave
// reads 512 contiguous bytes).  The block maximum is a quad reduction, every
// lane derives the block's scale from it (block_enc) and encodes its four
// elements with encode_one: the same fp32 steps as encode_block.  A launch of
// few blocks is bound by one thread's serial encode, which this cuts to a
// quarter.  Lane q of block b writes code bytes 2q, 2q + 1 of the block (the
// element order of encode_block), lane 0 the scale byte.
__global__ __launch_bounds__(kThreads) void k_quantize_quad(PackArgs a) {
    const float Sg = *a.sg_ptr;
    if (a.global_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *a.global_out = Sg;
    const float t = 6.0f * Sg;
    const int64_t nquad = a.rows * (a.cols / 4);   // a multiple of 4: quads of a block are whole
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const bool ok = i < nquad;
    const int64_t e = ok ? 4 * i : 0;
    const uint2 v = *reinterpret_cast<const uint2*>(a.x + e);
    uint32_t m = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
    m = max(m, dpp_u32<0xB1>(m));    // quad_perm [1,0,3,2]
    m = max(m, dpp_u32<0x4E>(m));    // quad_perm [2,3,0,1]: the block maximum
    const BlockEnc be = block_enc(m, Sg, t);
    const uint32_t c = encode_one(v.x, be) | (encode_one(v.x >> 16, be) << 4) | (encode_one(v.y, be) << 8) |
                       (encode_one(v.y >> 16, be) << 12);
    if (!ok) return;
    if (a.codes != nullptr) {
        reinterpret_cast<uint16_t*>(a.codes)[i] = (uint16_t)c;
        if ((i & 3) == 0) a.scales[i >> 2] = (uint8_t)be.s8;
    }
    if (a.xhat != nullptr) {
        // q * s for the 4 elements, exact in f16 and bf16
        const uint4 q = a.xhat_bf16 ? fp4x8_scaled_bf16_bits(c, be.s)
                                    : __builtin_bit_cast(uint4, fp4x8_scaled_f16(c, (_Float16)be.s));
        *reinterpret_cast<uint2*>(a.xhat + e) = make_uint2(q.x, q.y);
    }
}

// Dequantize: one piece of 8 elements (4 code bytes, half a block) per
// thread per step, two steps per iteration with both loads issued first.
// Consecutive threads take consecutive pieces, so every load and every
// 16-byte store of a wave is contiguous; non-temporal both ways (each byte is
// touched once).
__device__ __forceinline__ u32x4 dequant_piece(uint32_t c, uint32_t sbyte, float Sg) {
    const float s = e4m3_to_f32(sbyte);
    f32x2 q[4];
    fp4x8_to_f32(c, q);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float qs0 = q[i].x * s, qs1 = q[i].y * s;
        const float v0 = qs0 * Sg, v1 = qs1 * Sg;
        o[i] = f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

__global__ __launch_bounds__(kThreads) void k_dequantize(const uint32_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ sg_ptr,
                                                         float sg_const, int64_t npiece,
                                                         u32x4* __restrict__ y) {
    const float Sg = sg_ptr ? *sg_ptr : sg_const;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; p + stride < npiece; p += 2 * stride) {
        const uint32_t c0 = __builtin_nontemporal_load(codes + p);
        const uint32_t c1 = __builtin_nontemporal_load(codes + p + stride);
        const uint32_t s0 = __builtin_nontemporal_load(scales + (p >> 1));
        const uint32_t s1 = __builtin_nontemporal_load(scales + ((p + stride) >> 1));
        __builtin_nontemporal_store(dequant_piece(c0, s0, Sg), y + p);
        __builtin_nontemporal_store(dequant_piece(c1, s1, Sg), y + p + stride);
    }
    if (p < npiece) __builtin_nontemporal_store(dequant_piece(codes[p], scales[p >> 1], Sg), y + p);
}

// Packed NVFP4 -> the exact products q * s (no global scale) as f16 or bf16,
// one 8-element piece per thread per step: the operand form the GEMM and
// GEMV kernels consume.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_expand_qs(const uint32_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        int64_t npiece, uint4* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x; p < npiece; p += stride) {
        const uint32_t c = __builtin_nontemporal_load(codes + p);
        const float s = e4m3_to_f32(__builtin_nontemporal_load(scales + (p >> 1)));
        if constexpr (BF16) out[p] = fp4x8_scaled_bf16_bits(c, s);
        else out[p] = __builtin_bit_cast(uint4, fp4x8_scaled_f16(c, (_Float16)s));
    }
}

int grid_for(int64_t work, int per_block, int cap) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

}  // namespace

// Three 512-thread workgroups per CU: measured on 65536 x 6144, 768
// workgroups 114 us against 131 us with 1024 and 130 us with 512 (a thread's
// successive loads are grid x 8 KB apart: 6 MB rather than a power of two).
int amax_grid(int64_t n) { return grid_for(n / 8, kAmaxThreads * kAmaxUnroll, 768); }

// ----------------------------------------------------------- no-alloc scratch --
//
// Device memory of nvfp4_quantize_noalloc: the pass-1 partial maxima, at most
// kNoAllocPartials of them (amax_grid never exceeds 768).  Each GPU the
// library runs on holds its own copy until the process ends; every call on a
// GPU shares it, so calls that overlap on one GPU race (each call overwrites
// every entry it reads, so nothing needs clearing between calls).  Host code
// never passes the name `scratch` to a kernel: there it is a host-side
// stand-in, and the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint32_t scratch[kNoAllocPartials];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_partials(hipStream_t stream, uint32_t** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        // resolve the array's address once per device, with that device current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_amax_partial(const uint16_t* x, int64_t n, uint32_t* partial, int grid,
                               hipStream_t stream) {
    hipLaunchKernelGGL(k_amax_partial, dim3(grid), dim3(kAmaxThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), n / 8, partial);
    return hipGetLastError();
}

hipError_t launch_quantize_pack(const PackArgs& a, hipStream_t stream) {
    const int64_t nblk = a.rows * (a.cols / 16);
    if (a.mode == ScaleMode::kStatic && a.src_row == nullptr && a.rows_valid == nullptr && nblk > 0 &&
        nblk <= kQuadMaxBlocks) {
        hipLaunchKernelGGL(k_quantize_quad, dim3((unsigned)((4 * nblk + kThreads - 1) / kThreads)), dim3(kThreads),
                           0, stream, a);
        return hipGetLastError();
    }
    // two blocks per thread per iteration; 4096 workgroups measured best on
    // MI355X for 65536 x 6144 (202 against 212 us with 8192 and one block)
    const int grid = grid_for(nblk, kThreads * 2, 4096);
    switch (a.mode) {
        case ScaleMode::kDynamic:
            hipLaunchKernelGGL(k_quantize_pack<ScaleMode::kDynamic>, dim3(grid), dim3(kThreads), 0,
                               stream, a);
            break;
        case ScaleMode::kStatic:
            hipLaunchKernelGGL(k_quantize_pack<ScaleMode::kStatic>, dim3(grid), dim3(kThreads), 0,
                               stream, a);
            break;
        case ScaleMode::kGrouped:
            hipLaunchKernelGGL(k_quantize_pack<ScaleMode::kGrouped>, dim3(grid), dim3(kThreads), 0,
                               stream, a);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* sg_ptr,
                             float sg_const, int64_t rows, int64_t cols, uint16_t* y,
                             hipStream_t stream) {
    // about three pieces per thread (measured on MI355X: the store stream
    // wants tens of thousands of workgroups)
    const int64_t npiece = rows * (cols / 8);
    const int grid = grid_for(npiece, kThreads * 3, 65536);
    hipLaunchKernelGGL(k_dequantize, dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint32_t*>(codes), scales, sg_ptr, sg_const, npiece,
                       reinterpret_cast<u32x4*>(y));
    return hipGetLastError();
}

hipError_t launch_expand_qs(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                            uint16_t* out, bool bf16, hipStream_t stream) {
    const int64_t npiece = rows * (cols / 8);
    const int grid = grid_for(npiece, kThreads * 3, 65536);
    const uint32_t* c = reinterpret_cast<const uint32_t*>(codes);
    uint4* o = reinterpret_cast<uint4*>(out);
    if (bf16) hipLaunchKernelGGL(k_expand_qs<true>, dim3(grid), dim3(kThreads), 0, stream, c, scales, npiece, o);
    else hipLaunchKernelGGL(k_expand_qs<false>, dim3(grid), dim3(kThreads), 0, stream, c, scales, npiece, o);
    return hipGetLastError();
}

}  // namespace nvfp4
