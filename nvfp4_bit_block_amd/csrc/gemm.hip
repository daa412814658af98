// gemm.hip -- block-scaled NVFP4 GEMM tiles on gfx950 MFMA.
//
// Fprop Y = X * W^T with the contraction axis innermost on both operands
// ("Getting GLM-5.2 NVFP4 Post-Training off the ground", "Going deeper" and
// "TN, NT, and what actually binds").  Both operands are NVFP4 on the W4A4
// path (model card "vroomfondel/glm-5.2-reap-504B-v2-W4A4", "Kernel
// choice"); the W4A16 MoE path has bf16 activations.
//
// How the per-16 E4M3 scales are applied: gfx950's scaled MFMA takes one
// power-of-two scale per 32 elements, which cannot express a per-16 E4M3
// scale.  Instead every operand element is decoded to q * s, which is exact
// in f16 and in bf16 (<= 6 significant bits, range [2^-10, 2688]), and the
// tile is multiplied on v_mfma_f32_32x32x16_{f16,bf16} with fp32
// accumulation; the two global scales are applied once in the epilogue.
// The products are exact, so only the fp32 summation order differs from the
// plain definition.  W4A4 uses f16 operands (q * s in one packed f16 multiply
// per pair); bf16 activations use bf16 operands.
//
// Tile: BM x BN output, K step 64, 256 threads = 4 waves in a WM x WN grid,
// each wave owning (BM/WM) x (BN/WN) as 32x32 MFMA blocks.  Packed operands
// are prefetched into registers one K step ahead, decoded, and staged in LDS.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // 16-bit elements per LDS row (8 of padding)

template <AFmt AF>
struct OpType;
template <>
struct OpType<AFmt::kFp4> {
    using T = f16x8;
};
template <>
struct OpType<AFmt::kBf16> {
    using T = bf16x8;
};

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Packed 32-element unit (16 code bytes + 2 scale bytes) -> 32 16-bit values
// in LDS (four 16-byte stores).  f16 or bf16 per the MFMA operand type.
template <AFmt AF>
__device__ __forceinline__ void store_fp4_unit(uint16_t* dst, uint4 c, uint32_t s2, bool valid) {
    uint4* d = reinterpret_cast<uint4*>(dst);
    if (!valid) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        d[0] = z; d[1] = z; d[2] = z; d[3] = z;
        return;
    }
    const float s0 = e4m3_to_f32(s2 & 0xFFu), s1 = e4m3_to_f32((s2 >> 8) & 0xFFu);
    if constexpr (AF == AFmt::kFp4) {
        const _Float16 h0 = (_Float16)s0, h1 = (_Float16)s1;
        d[0] = __builtin_bit_cast(uint4, fp4x8_scaled_f16(c.x, h0));
        d[1] = __builtin_bit_cast(uint4, fp4x8_scaled_f16(c.y, h0));
        d[2] = __builtin_bit_cast(uint4, fp4x8_scaled_f16(c.z, h1));
        d[3] = __builtin_bit_cast(uint4, fp4x8_scaled_f16(c.w, h1));
    } else {
        d[0] = fp4x8_scaled_bf16_bits(c.x, s0);
        d[1] = fp4x8_scaled_bf16_bits(c.y, s0);
        d[2] = fp4x8_scaled_bf16_bits(c.z, s1);
        d[3] = fp4x8_scaled_bf16_bits(c.w, s1);
    }
}

template <int BM, int BN, int WM, int WN, AFmt AF, Epi EP>
__global__ __launch_bounds__(kThreads, 2) void k_gemm(GemmArgs g) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(WM * WN == 4 && TM >= 1 && TN >= 1, "tile");
    static_assert(EP != Epi::kMoeGateUp || (TN % 2) == 0, "gate/up needs paired column blocks");
    using OpT = typename OpType<AF>::T;

    __shared__ __align__(16) uint16_t As[BM * LDK];
    __shared__ __align__(16) uint16_t Bs[BN * LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // ---- which rows, columns, K range and group this workgroup owns
    int grp = 0;
    int64_t row_beg, row_end;
    if (g.groups > 0) {
        const int mt = (int)blockIdx.y;
        if (mt >= g.tile_off[g.groups]) return;
        int lo = 0, hi = g.groups;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (g.tile_off[mid] <= mt) lo = mid; else hi = mid;
        }
        grp = lo;
        row_beg = (int64_t)g.row_off[grp] + (int64_t)(mt - g.tile_off[grp]) * BM;
        row_end = min((int64_t)g.row_off[grp + 1], row_beg + BM);
    } else {
        row_beg = (int64_t)blockIdx.y * BM;
        row_end = min(g.M, row_beg + BM);
    }
    const int64_t kchunks = g.K / BK;
    const int64_t per = (kchunks + g.ksplit - 1) / g.ksplit;
    const int64_t kc0 = (int64_t)blockIdx.z * per;
    const int64_t kc1 = min(kchunks, kc0 + per);

    const int64_t KB = g.K / 2, KS = g.K / 16;  // bytes per row: codes, scales
    const uint8_t* bcodes = g.b_codes + (int64_t)grp * g.N * KB;
    const uint8_t* bscales = g.b_scales + (int64_t)grp * g.N * KS;

    // B row held in LDS row `rl`
    auto b_row = [&](int rl) -> int64_t {
        if constexpr (EP == Epi::kMoeGateUp) {
            const int w = rl / WTN, j = (rl % WTN) / 32, c = rl % 32;
            const int64_t j0 = (int64_t)blockIdx.x * (BN / 2) + w * (WTN / 2);
            return (j < TN / 2) ? j0 + j * 32 + c : g.half_n + j0 + (j - TN / 2) * 32 + c;
        } else {
            return (int64_t)blockIdx.x * BN + rl;
        }
    };
    const int64_t n_limit = g.N;

    // ---- per-thread load units: (row, half of the 64-wide K step)
    constexpr int A_UNITS = BM * 2, B_UNITS = BN * 2;
    const bool a_active = tid < A_UNITS;
    const bool b_active = tid < B_UNITS;
    const int a_rl = tid >> 1, a_half = tid & 1;
    const int b_rl = tid >> 1, b_half = tid & 1;
    const int64_t a_row = row_beg + a_rl;
    const bool a_valid = a_active && a_row < row_end;
    const int64_t b_grow = b_active ? b_row(b_rl) : 0;
    const bool b_valid = b_active && b_grow < n_limit;

    const uint8_t* a_src_c = nullptr;  // fp4 codes row
    const uint8_t* a_src_s = nullptr;
    const uint16_t* a_src_h = nullptr; // bf16 row
    if (a_valid) {
        if constexpr (AF == AFmt::kFp4) {
            a_src_c = reinterpret_cast<const uint8_t*>(g.a) + a_row * KB;
            a_src_s = g.a_scales + a_row * KS;
        } else {
            const int64_t src = g.a_rows ? (int64_t)(g.a_rows[a_row] / g.a_div) : a_row;
            a_src_h = reinterpret_cast<const uint16_t*>(g.a) + src * g.K;
        }
    }
    const uint8_t* b_src_c = b_valid ? bcodes + b_grow * KB : nullptr;
    const uint8_t* b_src_s = b_valid ? bscales + b_grow * KS : nullptr;

    // prefetch registers
    uint4 ra[4];
    uint32_t ras = 0;
    uint4 rb;
    uint32_t rbs = 0;

    auto load = [&](int64_t kc) {
        if (a_valid) {
            if constexpr (AF == AFmt::kFp4) {
                ra[0] = *reinterpret_cast<const uint4*>(a_src_c + kc * 32 + a_half * 16);
                ras = *reinterpret_cast<const uint16_t*>(a_src_s + kc * 4 + a_half * 2);
            } else {
                const uint4* p = reinterpret_cast<const uint4*>(a_src_h + kc * BK + a_half * 32);
                ra[0] = p[0]; ra[1] = p[1]; ra[2] = p[2]; ra[3] = p[3];
            }
        }
        if (b_valid) {
            rb = load_nt16(b_src_c + kc * 32 + b_half * 16);
            rbs = *reinterpret_cast<const uint16_t*>(b_src_s + kc * 4 + b_half * 2);
        }
    };
    auto stage = [&]() {
        if (a_active) {
            uint16_t* dst = &As[a_rl * LDK + a_half * 32];
            if constexpr (AF == AFmt::kFp4) {
                store_fp4_unit<AF>(dst, ra[0], ras, a_valid);
            } else {
                uint4* d = reinterpret_cast<uint4*>(dst);
                const uint4 z = make_uint4(0, 0, 0, 0);
                d[0] = a_valid ? ra[0] : z; d[1] = a_valid ? ra[1] : z;
                d[2] = a_valid ? ra[2] : z; d[3] = a_valid ? ra[3] : z;
            }
        }
        if (b_active) store_fp4_unit<AF>(&Bs[b_rl * LDK + b_half * 32], rb, rbs, b_valid);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (kc0 < kc1) load(kc0);
    for (int64_t kc = kc0; kc < kc1; ++kc) {
        stage();
        __syncthreads();
        if (kc + 1 < kc1) load(kc + 1);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            OpT af[TM], bf[TN];
            const int koff = kk * 16 + (lane >> 5) * 8;
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const OpT*>(&As[(wm * WTM + i * 32 + (lane & 31)) * LDK + koff]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *reinterpret_cast<const OpT*>(&Bs[(wn * WTN + j * 32 + (lane & 31)) * LDK + koff]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma(af[i], bf[j], acc[i][j]);
        }
        __syncthreads();
    }

    // ---- epilogue
    const int gi = g.groups > 0 ? grp : 0;
    const float sc = (g.a_global ? g.a_global[gi] : 1.0f) * (g.b_global ? g.b_global[gi] : 1.0f);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int il = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int64_t row = row_beg + il;
            if (row >= row_end) continue;
            if constexpr (EP == Epi::kMoeGateUp) {
#pragma unroll
                for (int j = 0; j < TN / 2; ++j) {
                    const int64_t hcol = (int64_t)blockIdx.x * (BN / 2) + wn * (WTN / 2) + j * 32 + (lane & 31);
                    if (hcol >= g.half_n) continue;
                    const float gv = acc[i][j][r] * sc;
                    const float uv = acc[i][j + TN / 2][r] * sc;
                    const float hv = gv / (1.0f + expf(-gv)) * uv;
                    reinterpret_cast<uint16_t*>(g.out)[row * g.ldo + hcol] = (uint16_t)f32_to_bf16_rne(hv);
                }
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t col = (int64_t)blockIdx.x * BN + wn * WTN + j * 32 + (lane & 31);
                    if (col >= g.N) continue;
                    const float v = acc[i][j][r];
                    if constexpr (EP == Epi::kStoreBf16) {
                        reinterpret_cast<uint16_t*>(g.out)[row * g.ldo + col] = (uint16_t)f32_to_bf16_rne(v * sc);
                    } else if constexpr (EP == Epi::kPartialF32) {
                        reinterpret_cast<float*>(g.out)[((int64_t)blockIdx.z * g.M + row) * g.ldo + col] = v;
                    } else {
                        reinterpret_cast<float*>(g.out)[row * g.ldo + col] = v * sc;
                    }
                }
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_splitk_reduce(const float* __restrict__ partial, int ksplit,
                                                            int64_t M, int64_t N, const float* __restrict__ g0,
                                                            const float* __restrict__ g1,
                                                            uint16_t* __restrict__ y) {
    const float scale = *g0 * (g1 ? *g1 : 1.0f);
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        float s = 0.0f;
        for (int k = 0; k < ksplit; ++k) s += partial[(int64_t)k * total + i];
        y[i] = (uint16_t)f32_to_bf16_rne(s * scale);
    }
}

template <int BM, int BN, int WM, int WN, AFmt AF, Epi EP>
hipError_t launch_cfg(const GemmArgs& g, int grid_m, hipStream_t stream) {
    int64_t ncols = (EP == Epi::kMoeGateUp) ? g.half_n : g.N;
    int64_t bn = (EP == Epi::kMoeGateUp) ? BN / 2 : BN;
    dim3 grid((unsigned)((ncols + bn - 1) / bn), (unsigned)grid_m, (unsigned)g.ksplit);
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, AF, EP>), grid, dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

template <AFmt AF, Epi EP>
hipError_t launch_tile(const GemmArgs& g, Tile tile, int grid_m, hipStream_t stream) {
    switch (tile) {
        case Tile::k128x128: return launch_cfg<128, 128, 2, 2, AF, EP>(g, grid_m, stream);
        case Tile::k64x128: return launch_cfg<64, 128, 2, 2, AF, EP>(g, grid_m, stream);
        case Tile::k32x128:
            if constexpr (EP == Epi::kMoeGateUp) return hipErrorInvalidValue;
            else return launch_cfg<32, 128, 1, 4, AF, EP>(g, grid_m, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, AFmt afmt, Epi epi, Tile tile, int grid_m,
                       hipStream_t stream) {
#define NVFP4_EPI(AF)                                                                   \
    switch (epi) {                                                                      \
        case Epi::kStoreBf16: return launch_tile<AF, Epi::kStoreBf16>(g, tile, grid_m, stream);   \
        case Epi::kPartialF32: return launch_tile<AF, Epi::kPartialF32>(g, tile, grid_m, stream); \
        case Epi::kMoeGateUp: return launch_tile<AF, Epi::kMoeGateUp>(g, tile, grid_m, stream);   \
        case Epi::kMoeDown: return launch_tile<AF, Epi::kMoeDown>(g, tile, grid_m, stream);       \
    }
    if (afmt == AFmt::kFp4) {
        NVFP4_EPI(AFmt::kFp4)
    } else {
        NVFP4_EPI(AFmt::kBf16)
    }
#undef NVFP4_EPI
    return hipErrorInvalidValue;
}

hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N,
                                const float* g0, const float* g1, uint16_t* y, hipStream_t stream) {
    int64_t grid = (M * N + kThreads - 1) / kThreads;
    if (grid > 8192) grid = 8192;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)grid), dim3(kThreads), 0, stream, partial,
                       ksplit, M, N, g0, g1, y);
    return hipGetLastError();
}

}  // namespace nvfp4
