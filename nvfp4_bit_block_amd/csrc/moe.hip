// moe.hip -- routing preparation and the weighted combine of the routed-expert
// layer ("GLM-5.2-NVFP4" model card: 256 routed experts, 8 per token).
//
// Routing ids and gate weights are inputs.  Routing runs in three launches:
// each workgroup counts the slots per expert of its own run of slots, one
// workgroup turns the counts into row offsets, bm-row tile offsets and every
// run's first row in each expert, and each workgroup then scatters its slots
// into its expert rows.  The row a slot lands on within its run may differ
// from run to run (LDS atomics), but every row is computed on its own, so the
// layer output does not depend on it.  The combine sums each token's slots in
// slot order in fp32.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kMaxExperts = 4096;

// Slots per routing workgroup: at least 1024, and few enough runs that the
// scan's per-expert walk over them stays short.
int64_t route_chunk(int64_t slots) {
    int64_t c = (slots + 1023) / 1024;
    c = (c + 255) / 256 * 256;
    return c < 1024 ? 1024 : c;
}

__global__ __launch_bounds__(kRouteThreads) void k_route_count(const int32_t* __restrict__ ids, int64_t slots,
                                                               int32_t E, int64_t chunk,
                                                               int32_t* __restrict__ counts) {
    __shared__ int32_t cnt[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kRouteThreads) cnt[e] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * chunk, p1 = min(slots, p0 + chunk);
    for (int64_t p = p0 + threadIdx.x; p < p1; p += kRouteThreads) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouteThreads) counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// counts [runs, E] -> base [runs, E]: each run's first row in each expert
// (row offsets included), row_off [E + 1], tile_off [E + 1].
__global__ __launch_bounds__(kScanThreads) void k_route_scan(const int32_t* __restrict__ counts, int runs,
                                                             int32_t E, int32_t bm, int32_t* __restrict__ base,
                                                             int32_t* __restrict__ row_off,
                                                             int32_t* __restrict__ tile_off) {
    __shared__ int32_t tot[kMaxExperts];
    __shared__ int32_t tiles[kMaxExperts];
    __shared__ int32_t part[2][kScanThreads];
    for (int e = threadIdx.x; e < E; e += kScanThreads) {
        // eight runs' counts in flight at a time
        int32_t r = 0;
        for (int g0 = 0; g0 < runs; g0 += 8) {
            int32_t c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = g0 + u < runs ? counts[(int64_t)(g0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (g0 + u < runs) base[(int64_t)(g0 + u) * E + e] = r;
                r += c[u];
            }
        }
        tot[e] = r;
        tiles[e] = (r + bm - 1) / bm;
    }
    __syncthreads();
    // exclusive scans over the experts: thread i sums its contiguous span,
    // the spans' sums are scanned across the block, then each span is walked
    const int span = (E + kScanThreads - 1) / kScanThreads;
    const int e0 = min(E, (int)threadIdx.x * span), e1 = min(E, e0 + span);
    int32_t sr = 0, st = 0;
    for (int e = e0; e < e1; ++e) {
        sr += tot[e];
        st += tiles[e];
    }
    part[0][threadIdx.x] = sr;
    part[1][threadIdx.x] = st;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int32_t a = threadIdx.x >= off ? part[0][threadIdx.x - off] : 0;
        const int32_t b = threadIdx.x >= off ? part[1][threadIdx.x - off] : 0;
        __syncthreads();
        part[0][threadIdx.x] += a;
        part[1][threadIdx.x] += b;
        __syncthreads();
    }
    int32_t r = part[0][threadIdx.x] - sr, t = part[1][threadIdx.x] - st;   // exclusive
    for (int e = e0; e < e1; ++e) {
        row_off[e] = r;
        tile_off[e] = t;
        r += tot[e];
        t += tiles[e];
    }
    if (threadIdx.x == kScanThreads - 1) {
        row_off[E] = part[0][kScanThreads - 1];
        tile_off[E] = part[1][kScanThreads - 1];
    }
}

__global__ __launch_bounds__(kRouteThreads) void k_route_scatter(const int32_t* __restrict__ ids, int64_t slots,
                                                                 int32_t E, int64_t chunk,
                                                                 const int32_t* __restrict__ base,
                                                                 const int32_t* __restrict__ row_off,
                                                                 int32_t* __restrict__ perm,
                                                                 int32_t* __restrict__ inv,
                                                                 int32_t* __restrict__ pos_group) {
    __shared__ int32_t cur[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kRouteThreads) cur[e] = row_off[e] + base[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * chunk, p1 = min(slots, p0 + chunk);
    for (int64_t p = p0 + threadIdx.x; p < p1; p += kRouteThreads) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E) {
            const int32_t pos = atomicAdd(&cur[e], 1);
            perm[pos] = (int32_t)p;
            inv[p] = pos;
            pos_group[pos] = e;
        } else {
            inv[p] = -1;
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

size_t moe_route_scratch_bytes(int64_t slots, int32_t E) {
    const int64_t runs = slots > 0 ? (slots + route_chunk(slots) - 1) / route_chunk(slots) : 1;
    return (size_t)(2 * runs * E) * 4;
}

hipError_t launch_moe_route(const int32_t* ids, int64_t slots, int32_t E, int32_t bm,
                            int32_t* row_off, int32_t* tile_off, int32_t* perm, int32_t* inv,
                            int32_t* pos_group, int32_t* scratch, hipStream_t stream) {
    if (E < 1 || E > kMaxExperts || bm < 1) return hipErrorInvalidValue;
    const int64_t chunk = route_chunk(slots);
    const int64_t runs = slots > 0 ? (slots + chunk - 1) / chunk : 1;
    int32_t* counts = scratch;
    int32_t* base = scratch + runs * E;
    hipLaunchKernelGGL(k_route_count, dim3((unsigned)runs), dim3(kRouteThreads), 0, stream, ids, slots, E, chunk,
                       counts);
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(kScanThreads), 0, stream, counts, (int)runs, E, bm, base,
                       row_off, tile_off);
    hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)runs), dim3(kRouteThreads), 0, stream, ids, slots, E, chunk,
                       base, row_off, perm, inv, pos_group);
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
