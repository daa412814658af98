// gemm_st.hip -- W4A4 NVFP4 GEMM with packed operands staged in LDS.
//
// Fprop Y = X * W^T with the contraction axis innermost on both operands
// ("Getting GLM-5.2 NVFP4 Post-Training off the ground", "Going deeper" and
// "TN, NT, and what actually binds"); both operands NVFP4 per the model card
// "vroomfondel/glm-5.2-reap-504B-v2-W4A4", "Kernel choice".
//
// Scale application: every operand element is decoded to q * s, exact in f16,
// and multiplied on v_mfma_f32_32x32x16_f16 with fp32 accumulation; the two
// global scales are applied in the epilogue.  (gfx950's scaled MFMA takes one
// power-of-two scale per 32 elements and its fp4 conversions use only the
// exponent of their scale operand: neither can carry a per-16 E4M3 scale.)
//
// Data movement.  The workgroup copies packed codes and scale bytes, still
// NVFP4, from global memory through registers into LDS, four 64-wide K steps
// (128 code bytes and 16 scale bytes per row) per stage, double-buffered.
// Consecutive lanes fetch consecutive 16-byte chunks of a row, so each load
// instruction touches few cache lines.  Each wave then reads its rows'
// fragments from LDS, decodes them in registers and issues the MFMAs; only
// packed data crosses LDS (0.5625 byte per element and operand).
//
// K order inside a 64-wide K step: the 32x32x16 MFMA takes, in lane l, row
// (or column) l % 32 and 8 consecutive K positions selected by l / 32.  A K
// permutation applied to both operands leaves the product unchanged, so lane
// half hf = l / 32 takes K positions [32 hf, 32 hf + 32) of the step (16
// contiguous code bytes and two scale bytes) and MFMA kk of the step uses
// positions 32 hf + 8 kk + [0, 8).
//
// LDS layout per stage: [A rows; B rows] x 144 bytes of codes (128 + 16 of
// padding: a row stride of 36 dwords keeps the 16-byte reads of 16
// consecutive rows on distinct banks), then [A rows; B rows] x 16 scale bytes.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data, range checked
constexpr uint32_t kOob = 0x80000000u;  // an offset past every buffer built here

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes) {
    const uint32_t n = bytes < 0x80000000ull ? (uint32_t)bytes : 0x80000000u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int kk) {
    return kk == 0 ? v.x : kk == 1 ? v.y : kk == 2 ? v.z : v.w;
}

constexpr int kStepsPerStage = 4;
constexpr int kRowCode = 144;  // LDS bytes per row of codes per stage (128 + pad)
constexpr int kRowScale = 16;  // LDS bytes per row of scales per stage
constexpr int kGroupM = 8;     // m-tiles per band in the ungrouped tile order

template <int TM, int TN, int WM, int WN>
struct StCfg {
    static constexpr int NW = WM * WN, NT = 64 * NW;
    static constexpr int WTM = 32 * TM, WTN = 32 * TN;
    static constexpr int BM = WTM * WM, BN = WTN * WN, ROWS = BM + BN;
    static constexpr int CODE_BYTES = ROWS * kRowCode, SCALE_BYTES = ROWS * kRowScale;
    static constexpr int STAGE = CODE_BYTES + SCALE_BYTES;
    static constexpr int JC = CODE_BYTES / 1024;  // code copy jobs (1 KB each)
    static constexpr int JS = SCALE_BYTES / 1024; // scale copy jobs (64 rows each)
    static constexpr int JOBS = JC + JS;
    static constexpr int JPW = (JOBS + NW - 1) / NW;  // jobs per wave
    static_assert(BM % 64 == 0 && BN % 64 == 0, "copy jobs must not straddle the A/B boundary");
    static_assert(CODE_BYTES % 1024 == 0 && SCALE_BYTES % 1024 == 0, "whole jobs");
    static_assert(2 * STAGE <= 160 * 1024, "LDS");
};

template <int TM, int TN, int WM, int WN, Epi EP>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_st(GemmArgs g) {
    using C = StCfg<TM, TN, WM, WN>;
    constexpr int BM = C::BM, BN = C::BN, WTM = C::WTM, WTN = C::WTN;
    static_assert(EP != Epi::kMoeGateUp || (TN % 2) == 0, "gate/up needs paired column blocks");
    __shared__ __align__(16) uint8_t smem[2 * C::STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int c32 = lane & 31, hf = lane >> 5;

    // ---- tile, group and K range of this workgroup
    int grp = 0, tn, kz;
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
        tn = (int)blockIdx.x;
        kz = (int)blockIdx.z;
    } else {
        // Workgroups are dealt to the 8 XCDs round-robin by linear id; renumber
        // so that each XCD receives a contiguous run of tiles, and walk tiles in
        // bands of kGroupM m-tiles so that concurrently running tiles share rows
        // of A and columns of B in that XCD's L2.
        const int nwg = (int)gridDim.x;
        int id = (int)blockIdx.x;
        if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
        const int mtiles = (int)((g.M + BM - 1) / BM);
        const int ntiles = (int)((g.N + BN - 1) / BN);
        const int per_split = mtiles * ntiles;
        kz = id / per_split;
        const int t = id - kz * per_split;
        const int band = t / (kGroupM * ntiles);
        const int first_m = band * kGroupM;
        const int gsz = min(mtiles - first_m, kGroupM);
        const int r = t - band * kGroupM * ntiles;
        const int tm = first_m + r % gsz;
        tn = r / gsz;
        row_beg = (int64_t)tm * BM;
        row_end = min(g.M, row_beg + BM);
    }
    // K range of this split in stages of 4 steps (K % 256 == 0 on this path)
    const int nstage_all = (int)(g.K / (64 * kStepsPerStage));
    const int per = (nstage_all + g.ksplit - 1) / g.ksplit;
    const int st0 = __builtin_amdgcn_readfirstlane(kz * per);
    const int nst = __builtin_amdgcn_readfirstlane(max(0, min(nstage_all - st0, per)));

    const uint32_t KB = (uint32_t)(g.K / 2), KS = (uint32_t)(g.K / 16);
    const int64_t nrows = row_end - row_beg;
    const Rsrc ra_c = make_rsrc(reinterpret_cast<const uint8_t*>(g.a) + row_beg * KB, (uint64_t)nrows * KB);
    const Rsrc ra_s = make_rsrc(g.a_scales + row_beg * KS, (uint64_t)nrows * KS);
    const Rsrc rb_c = make_rsrc(g.b_codes + (int64_t)grp * g.N * KB, (uint64_t)g.N * KB);
    const Rsrc rb_s = make_rsrc(g.b_scales + (int64_t)grp * g.N * KS, (uint64_t)g.N * KS);

    // Global column of B row n of the tile (or -1 when past the end).
    auto b_col = [&](int n) -> int64_t {
        if constexpr (EP == Epi::kMoeGateUp) {
            // column block j of wave w: gate columns for j < TN/2, the matching
            // up columns (I further) for j >= TN/2
            const int w = n / WTN, j = (n % WTN) / 32, cc = n % 32;
            const int jj = j % (TN / 2 > 0 ? TN / 2 : 1);
            const int64_t hcol = (int64_t)tn * (BN / 2) + w * (WTN / 2) + 32 * jj + cc;
            if (hcol >= g.half_n) return -1;
            return (j < TN / 2) ? hcol : g.half_n + hcol;
        } else {
            const int64_t col = (int64_t)tn * BN + n;
            return col < g.N ? col : -1;
        }
    };

    // ---- this lane's source offsets for each of the wave's copy jobs
    uint32_t jvoff[C::JPW];
#pragma unroll
    for (int k = 0; k < C::JPW; ++k) {
        int j = wave + k * C::NW;
        if (j >= C::JOBS) j = wave;  // surplus slot: repeat a job (same bytes, same place)
        uint32_t v = kOob;
        if (j < C::JC) {
            const int p = j * 64 + lane;       // 16-byte chunk of the padded code region
            const int q = p / 9, cc = p % 9;   // row, chunk (chunk 8 is padding)
            if (cc < 8) {
                if (q < BM) {
                    v = (uint32_t)q * KB + 16u * cc;
                } else {
                    const int64_t col = b_col(q - BM);
                    if (col >= 0) v = (uint32_t)col * KB + 16u * cc;
                }
            }
        } else {
            const int q = (j - C::JC) * 64 + lane;
            if (q < BM) {
                v = (uint32_t)q * KS;
            } else {
                const int64_t col = b_col(q - BM);
                if (col >= 0) v = (uint32_t)col * KS;
            }
        }
        jvoff[k] = v;
    }

    // A stage is fetched into registers (one 16-byte chunk per lane and job)
    // while the previous stage is multiplied, then written to LDS.
    uint4 stg[C::JPW];
    auto load_stage = [&](int st) {
#pragma unroll
        for (int k = 0; k < C::JPW; ++k) {
            int j = wave + k * C::NW;
            if (j >= C::JOBS) j = wave;
            // (branches, not selects, between the descriptors: the job kind is
            // uniform, and a select of descriptors would go through memory)
            if (j < C::JC) {
                if ((j * 64) / 9 < BM) stg[k] = bload16(ra_c, jvoff[k], (uint32_t)st * 128u);
                else stg[k] = bload16(rb_c, jvoff[k], (uint32_t)st * 128u);
            } else {
                if ((j - C::JC) * 64 < BM) stg[k] = bload16(ra_s, jvoff[k], (uint32_t)st * 16u);
                else stg[k] = bload16(rb_s, jvoff[k], (uint32_t)st * 16u);
            }
        }
    };
    auto store_stage = [&](int buf) {
        uint8_t* base = smem + buf * C::STAGE;
#pragma unroll
        for (int k = 0; k < C::JPW; ++k) {
            int j = wave + k * C::NW;
            if (j >= C::JOBS) j = wave;  // surplus slot: the same bytes to the same place
            uint8_t* dst = (j < C::JC) ? base + j * 1024 : base + C::CODE_BYTES + (j - C::JC) * 1024;
            *reinterpret_cast<uint4*>(dst + 16 * lane) = stg[k];
        }
    };

    // ---- fragment addresses (within a stage buffer)
    uint32_t a_code[TM], a_scale[TM], b_code[TN], b_scale[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int q = wm * WTM + 32 * i + c32;
        a_code[i] = q * kRowCode + 16 * hf;
        a_scale[i] = C::CODE_BYTES + q * kRowScale;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int q = BM + wn * WTN + 32 * j + c32;
        b_code[j] = q * kRowCode + 16 * hf;
        b_scale[j] = C::CODE_BYTES + q * kRowScale;
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto compute_stage = [&](int buf) {
        const uint8_t* base = smem + buf * C::STAGE;
#pragma unroll
        for (int t = 0; t < kStepsPerStage; ++t) {
            uint4 ca[TM], cb[TN];
            uint32_t sa[TM], sb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                ca[i] = *reinterpret_cast<const uint4*>(base + a_code[i] + 32 * t);
                sa[i] = *reinterpret_cast<const uint32_t*>(base + a_scale[i] + 4 * t);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                cb[j] = *reinterpret_cast<const uint4*>(base + b_code[j] + 32 * t);
                sb[j] = *reinterpret_cast<const uint32_t*>(base + b_scale[j] + 4 * t);
            }
            f32x2 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = e4m3x2_to_f32(sa[i] >> (16 * hf));
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = e4m3x2_to_f32(sb[j] >> (16 * hf));
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                f16x8 av[TM], bv[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    av[i] = fp4x8_scaled_f16(word(ca[i], kk), (_Float16)(kk < 2 ? fa[i].x : fa[i].y));
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bv[j] = fp4x8_scaled_f16(word(cb[j], kk), (_Float16)(kk < 2 ? fb[j].x : fb[j].y));
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma(av[i], bv[j], acc[i][j]);
            }
        }
    };

    // ---- main loop: one barrier per stage.  Iteration s multiplies buffer
    // s % 2 while the loads of stage s + 1 are in flight, then writes stage
    // s + 1 into the other buffer (last read in iteration s - 1, before the
    // previous barrier) and starts the loads of stage s + 2.
    if (nst > 0) {
        load_stage(st0);
        store_stage(0);
        if (nst > 1) load_stage(st0 + 1);
        __syncthreads();
    }
    for (int s = 0; s < nst; ++s) {
        compute_stage(s & 1);
        if (s + 1 < nst) {
            store_stage((s + 1) & 1);
            if (s + 2 < nst) load_stage(st0 + s + 2);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds rows 8 (r/4) + 4 hf + r%4 of each 32x32 block, column c32
    const int gi = g.groups > 0 ? grp : 0;
    const float sc = (g.a_global ? g.a_global[gi] : 1.0f) * (g.b_global ? g.b_global[gi] : 1.0f);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = row_beg + wm * WTM + 32 * i + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (row >= row_end) continue;
            if constexpr (EP == Epi::kMoeGateUp) {
#pragma unroll
                for (int j = 0; j < TN / 2; ++j) {
                    const int64_t hcol = (int64_t)tn * (BN / 2) + wn * (WTN / 2) + 32 * j + c32;
                    if (hcol >= g.half_n) continue;
                    const float gv = acc[i][j][r] * sc;
                    const float uv = acc[i][j + TN / 2][r] * sc;
                    const float hv = gv / (1.0f + expf(-gv)) * uv;
                    reinterpret_cast<uint16_t*>(g.out)[row * g.ldo + hcol] = (uint16_t)f32_to_bf16_rne(hv);
                }
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t col = (int64_t)tn * BN + wn * WTN + 32 * j + c32;
                    if (col >= g.N) continue;
                    const float v = acc[i][j][r];
                    if constexpr (EP == Epi::kStoreBf16) {
                        reinterpret_cast<uint16_t*>(g.out)[row * g.ldo + col] = (uint16_t)f32_to_bf16_rne(v * sc);
                    } else if constexpr (EP == Epi::kPartialF32) {
                        reinterpret_cast<float*>(g.out)[((int64_t)kz * g.M + row) * g.ldo + col] = v;
                    } else {
                        reinterpret_cast<float*>(g.out)[row * g.ldo + col] = v * sc;
                    }
                }
            }
        }
    }
}

template <int TM, int TN, int WM, int WN, Epi EP>
hipError_t launch_cfg(const GemmArgs& g, int grid_m, hipStream_t stream) {
    using C = StCfg<TM, TN, WM, WN>;
    dim3 grid;
    if (g.groups > 0) {
        const int64_t ncols = (EP == Epi::kMoeGateUp) ? g.half_n : g.N;
        const int64_t bn = (EP == Epi::kMoeGateUp) ? C::BN / 2 : C::BN;
        grid = dim3((unsigned)((ncols + bn - 1) / bn), (unsigned)grid_m, (unsigned)g.ksplit);
    } else {
        const int64_t tiles = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN) * g.ksplit;
        grid = dim3((unsigned)tiles);
    }
    hipLaunchKernelGGL((k_gemm_st<TM, TN, WM, WN, EP>), grid, dim3(C::NT), 0, stream, g);
    return hipGetLastError();
}

template <Epi EP>
hipError_t launch_st_tile(const GemmArgs& g, StTile tile, int grid_m, hipStream_t stream) {
    switch (tile) {
        case StTile::k256x256_w128x128: return launch_cfg<4, 4, 2, 2, EP>(g, grid_m, stream);
        case StTile::k256x256_w128x64: return launch_cfg<4, 2, 2, 4, EP>(g, grid_m, stream);
        case StTile::k256x128_w128x64: return launch_cfg<4, 2, 2, 2, EP>(g, grid_m, stream);
        case StTile::k128x256_w128x64: return launch_cfg<4, 2, 1, 4, EP>(g, grid_m, stream);
        case StTile::k128x128_w64x64: return launch_cfg<2, 2, 2, 2, EP>(g, grid_m, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int st_tile_rows(StTile t) {
    switch (t) {
        case StTile::k256x256_w128x128: return 256;
        case StTile::k256x256_w128x64: return 256;
        case StTile::k256x128_w128x64: return 256;
        case StTile::k128x256_w128x64: return 128;
        case StTile::k128x128_w64x64: return 128;
    }
    return 0;
}

int st_tile_cols(StTile t) {
    switch (t) {
        case StTile::k256x256_w128x128: return 256;
        case StTile::k256x256_w128x64: return 256;
        case StTile::k256x128_w128x64: return 128;
        case StTile::k128x256_w128x64: return 256;
        case StTile::k128x128_w64x64: return 128;
    }
    return 0;
}

hipError_t launch_gemm_st(const GemmArgs& g, Epi epi, StTile tile, int grid_m, hipStream_t stream) {
    switch (epi) {
        case Epi::kStoreBf16: return launch_st_tile<Epi::kStoreBf16>(g, tile, grid_m, stream);
        case Epi::kPartialF32: return launch_st_tile<Epi::kPartialF32>(g, tile, grid_m, stream);
        case Epi::kMoeGateUp: return launch_st_tile<Epi::kMoeGateUp>(g, tile, grid_m, stream);
        case Epi::kMoeDown: return launch_st_tile<Epi::kMoeDown>(g, tile, grid_m, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace nvfp4
