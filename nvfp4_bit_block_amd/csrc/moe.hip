// moe.hip -- routing preparation and the weighted combine of the routed-expert
// layer ("GLM-5.2-NVFP4" model card: 256 routed experts, 8 per token).
//
// Routing ids and gate weights are inputs.  One workgroup counts the slots per
// expert, scans the counts into row offsets and bm-row tile offsets, and
// scatters every (token, slot) into its expert's contiguous rows.  The row a
// slot lands on may differ from run to run (LDS atomics), but every row is
// computed on its own, so the layer output does not depend on it.  The
// combine sums each token's slots in slot order in fp32.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteBatch = 8;
constexpr int kMaxExperts = 4096;

__global__ __launch_bounds__(kRouteThreads) void k_moe_route(const int32_t* __restrict__ ids,
                                                             int64_t slots, int32_t E, int32_t bm,
                                                             int32_t* __restrict__ row_off,
                                                             int32_t* __restrict__ tile_off,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv,
                                                             int32_t* __restrict__ pos_group) {
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t cur[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kRouteThreads) cnt[e] = 0;
    __syncthreads();
    // the slot loops issue kRouteBatch id loads before their atomics, so a
    // thread waits on memory once per batch rather than once per slot
    for (int64_t p0 = threadIdx.x; p0 < slots; p0 += (int64_t)kRouteThreads * kRouteBatch) {
        int32_t e[kRouteBatch];
#pragma unroll
        for (int u = 0; u < kRouteBatch; ++u) {
            const int64_t p = p0 + (int64_t)u * kRouteThreads;
            e[u] = p < slots ? ids[p] : -1;
        }
#pragma unroll
        for (int u = 0; u < kRouteBatch; ++u)
            if (e[u] >= 0 && e[u] < E) atomicAdd(&cnt[e[u]], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t r = 0, t = 0;
        for (int e = 0; e < E; ++e) {
            row_off[e] = r;
            tile_off[e] = t;
            cur[e] = r;
            r += cnt[e];
            t += (cnt[e] + bm - 1) / bm;
        }
        row_off[E] = r;
        tile_off[E] = t;
    }
    __syncthreads();
    for (int64_t p0 = threadIdx.x; p0 < slots; p0 += (int64_t)kRouteThreads * kRouteBatch) {
        int32_t e[kRouteBatch];
#pragma unroll
        for (int u = 0; u < kRouteBatch; ++u) {
            const int64_t p = p0 + (int64_t)u * kRouteThreads;
            e[u] = p < slots ? ids[p] : -1;
        }
#pragma unroll
        for (int u = 0; u < kRouteBatch; ++u) {
            const int64_t p = p0 + (int64_t)u * kRouteThreads;
            if (p >= slots) break;
            if (e[u] >= 0 && e[u] < E) {
                const int32_t pos = atomicAdd(&cur[e[u]], 1);
                perm[pos] = (int32_t)p;
                inv[p] = pos;
                pos_group[pos] = e[u];
            } else {
                inv[p] = -1;
            }
        }
    }
}

// out[t, n] = bf16(sum_j w[t, j] * Y[inv[t*k + j], n]); four columns per thread.
__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ Y,
                                                     const int32_t* __restrict__ inv,
                                                     const float* __restrict__ w, int64_t T,
                                                     int32_t topk, int64_t H,
                                                     uint16_t* __restrict__ out) {
    const int64_t h4 = H / 4;
    const int64_t total = T * h4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t t = i / h4, c = (i - t * h4) * 4;
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
        // slots in order, eight at a time: all eight row loads are issued
        // before the first sum (dropped slots load row 0 and are not added)
        for (int j0 = 0; j0 < topk; j0 += 8) {
            int32_t pos[8];
            float wj[8];
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const bool in = j0 + u < topk;
                pos[u] = in ? inv[t * topk + j0 + u] : -1;
                wj[u] = in ? w[t * topk + j0 + u] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4*>(Y + (int64_t)(pos[u] < 0 ? 0 : pos[u]) * H + c));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (pos[u] < 0) continue;
                s0 = __builtin_fmaf(wj[u], v[u][0], s0);
                s1 = __builtin_fmaf(wj[u], v[u][1], s1);
                s2 = __builtin_fmaf(wj[u], v[u][2], s2);
                s3 = __builtin_fmaf(wj[u], v[u][3], s3);
            }
        }
        const uint32_t lo = f32_to_bf16_rne(s0) | (f32_to_bf16_rne(s1) << 16);
        const uint32_t hi = f32_to_bf16_rne(s2) | (f32_to_bf16_rne(s3) << 16);
        *reinterpret_cast<uint2*>(out + t * H + c) = make_uint2(lo, hi);
    }
}

}  // namespace

hipError_t launch_moe_route(const int32_t* ids, int64_t slots, int32_t E, int32_t bm,
                            int32_t* row_off, int32_t* tile_off, int32_t* perm, int32_t* inv,
                            int32_t* pos_group, hipStream_t stream) {
    if (E > kMaxExperts) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(kRouteThreads), 0, stream, ids, slots, E, bm,
                       row_off, tile_off, perm, inv, pos_group);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float* Y, const int32_t* inv, const float* w, int64_t T,
                              int32_t topk, int64_t H, uint16_t* out, hipStream_t stream) {
    int64_t grid = (T * (H / 4) + 255) / 256;
    if (grid > 16384) grid = 16384;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)grid), dim3(256), 0, stream, Y, inv, w, T,
                       topk, H, out);
    return hipGetLastError();
}

}  // namespace nvfp4
