// hbm_probe.hip -- HBM read ceiling of one launch, for the benchmark's
// roofline: a kernel that only streams a buffer from HBM (16-byte
// non-temporal loads, every load instruction of a wave covering 1 KB
// contiguous, U loads in flight per thread), XORs what it reads and writes
// one word per workgroup so the loads cannot be dropped.  It bounds what any
// kernel that reads the same bytes in one launch can reach on this GPU.
// Not part of the NVFP4 library: a separate shared object that only the
// benchmark loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(512) void k_stream_read(const u32x4* __restrict__ p, int64_t n16, uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * 512;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * 512 + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[8];
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < 8; ++w) r ^= red[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace

extern "C" int32_t nvfp4probe_stream_read(const void* buf, int64_t bytes, int32_t workgroups, int32_t unroll,
                                          uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65536) return 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const u32x4* p = reinterpret_cast<const u32x4*>(buf);
    switch (unroll) {
        case 2: hipLaunchKernelGGL(k_stream_read<2>, dim3(workgroups), dim3(512), 0, s, p, bytes / 16, sink); break;
        case 4: hipLaunchKernelGGL(k_stream_read<4>, dim3(workgroups), dim3(512), 0, s, p, bytes / 16, sink); break;
        case 8: hipLaunchKernelGGL(k_stream_read<8>, dim3(workgroups), dim3(512), 0, s, p, bytes / 16, sink); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 6;
}
