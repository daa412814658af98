// gemm_rd.hip -- NVFP4 GEMM with operands fed from global memory straight
// into MFMA registers (no LDS staging, no workgroup barriers).
//
// Fprop Y = X * W^T with the contraction axis innermost on both operands
// ("Getting GLM-5.2 NVFP4 Post-Training off the ground", "Going deeper" and
// "TN, NT, and what actually binds"); W4A4 and W4A16 per the model card
// "vroomfondel/glm-5.2-reap-504B-v2-W4A4", "Kernel choice".
//
// Scale application: every operand element is decoded to q * s, exact in f16
// (W4A4) or bf16 (bf16 activations), and multiplied on
// v_mfma_f32_32x32x16_{f16,bf16} with fp32 accumulation; the global scales
// are applied in the epilogue.  (gfx950's own scaled MFMA takes power-of-two
// scales per 32 elements, and its fp4 conversions use only the exponent of
// their scale operand, so neither can carry a per-16 E4M3 scale.)
//
// K order inside a 64-wide K step.  The 32x32x16 MFMA takes, in lane l, row
// (or column) l % 32 and 8 consecutive K positions selected by l / 32.  Any
// permutation of K applied to both operands leaves the product unchanged, so
// lane half hf = l / 32 is given K positions [32 hf, 32 hf + 32) of the step
// and MFMA kk of the step consumes positions 32 hf + 8 kk + [0, 8).  A lane's
// share of a row is then 16 contiguous code bytes (32 elements) and two
// scale bytes, loaded with one 16-byte and one 4-byte buffer load per 64-wide
// K step and per 32-row block.  Rows or columns past the end read as zero
// through the buffer range check.
//
// Workgroup: WM x WN waves, each owning (32 TM) x (32 TN) outputs; the
// workgroup tile is (32 TM WM) x (32 TN WN).  Loads run one K step ahead of
// the MFMAs (two register sets used in turn).
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data, range checked
constexpr uint32_t kOob = 0x80000000u;  // an offset past every buffer this file builds

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes) {
    const uint32_t n = bytes < 0x80000000ull ? (uint32_t)bytes : 0x80000000u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload4(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A lane's packed share of one 32-row block for one K step: 32 codes and the
// step's four scale bytes (the lane uses bytes 2 hf and 2 hf + 1).
struct Fp4Frag {
    uint4 c;
    uint32_t s;
};
// A lane's share as 16-bit values (bf16, or f16 products q * s): 32 values.
struct WideFrag {
    uint4 v[4];
};

template <AFmt AF>
struct ATraits;
template <>
struct ATraits<AFmt::kFp4> {
    using Frag = Fp4Frag;
    using Op = f16x8;
};
template <>
struct ATraits<AFmt::kBf16> {
    using Frag = WideFrag;
    using Op = bf16x8;
};
template <>
struct ATraits<AFmt::kF16> {
    using Frag = WideFrag;
    using Op = f16x8;
};

// The lane's two block scales of a K step, as fp32 (exact).
__device__ __forceinline__ f32x2 frag_scales(uint32_t s4, int hf) {
    return e4m3x2_to_f32(s4 >> (16 * hf));
}

template <typename Op>
__device__ __forceinline__ Op decode(uint32_t w, float s);
template <>
__device__ __forceinline__ f16x8 decode<f16x8>(uint32_t w, float s) {
    return fp4x8_scaled_f16(w, (_Float16)s);
}
template <>
__device__ __forceinline__ bf16x8 decode<bf16x8>(uint32_t w, float s) {
    return __builtin_bit_cast(bf16x8, fp4x8_scaled_bf16_bits(w, s));
}

__device__ __forceinline__ uint32_t word(const uint4& v, int kk) {
    return kk == 0 ? v.x : kk == 1 ? v.y : kk == 2 ? v.z : v.w;
}

constexpr int kGroupM = 8;  // m-tiles per band in the ungrouped tile order

template <int TM, int TN, int WM, int WN, AFmt AF, Epi EP>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_rd(GemmArgs g) {
    constexpr int WTM = 32 * TM, WTN = 32 * TN;
    constexpr int BM = WTM * WM, BN = WTN * WN;
    static_assert(EP != Epi::kMoeGateUp || (TN % 2) == 0, "gate/up needs paired column blocks");
    using AFrag = typename ATraits<AF>::Frag;
    using Op = typename ATraits<AF>::Op;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int c = lane & 31, hf = lane >> 5;

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
    // K range of this split, kept in scalar registers (the buffer loads take
    // the step offset as their scalar operand).
    const int ksteps = (int)(g.K / 64);
    const int per = (ksteps + g.ksplit - 1) / g.ksplit;
    const int kc0 = __builtin_amdgcn_readfirstlane(kz * per);
    const int nsteps = __builtin_amdgcn_readfirstlane(max(0, min(ksteps - kc0, per)));

    const uint32_t KB = (uint32_t)(g.K / 2), KS = (uint32_t)(g.K / 16);
    const int64_t nrows = row_end - row_beg;

    // ---- A operand resources and per-lane offsets
    Rsrc ra_c, ra_s;
    uint32_t va_c[TM], va_s[TM];
    if constexpr (AF == AFmt::kFp4) {
        ra_c = make_rsrc(reinterpret_cast<const uint8_t*>(g.a) + row_beg * KB, (uint64_t)nrows * KB);
        ra_s = make_rsrc(g.a_scales + row_beg * KS, (uint64_t)nrows * KS);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t rl = (uint32_t)(wm * WTM + 32 * i + c);
            va_c[i] = rl * KB + 16u * hf;
            va_s[i] = rl * KS;
        }
    } else {
        // 16-bit rows, optionally gathered: one resource over the whole tensor
        // (the host checks that it spans less than 2 GiB).
        ra_c = make_rsrc(g.a, (uint64_t)g.a_src_rows * (uint64_t)g.K * 2);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t r = row_beg + wm * WTM + 32 * i + c;
            if (r < row_end) {
                const int64_t src = g.a_rows ? (int64_t)(g.a_rows[r] / g.a_div) : r;
                va_c[i] = (uint32_t)(src * g.K * 2) + 64u * hf;
            } else {
                va_c[i] = kOob;
            }
            va_s[i] = 0;
        }
    }

    // ---- B operand (NVFP4 [N, K] of this group)
    const Rsrc rb_c = make_rsrc(g.b_codes + (int64_t)grp * g.N * KB, (uint64_t)g.N * KB);
    const Rsrc rb_s = make_rsrc(g.b_scales + (int64_t)grp * g.N * KS, (uint64_t)g.N * KS);
    uint32_t vb_c[TN], vb_s[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        int64_t col;
        bool ok;
        if constexpr (EP == Epi::kMoeGateUp) {
            const int jj = j % (TN / 2 > 0 ? TN / 2 : 1);
            const int64_t hcol = (int64_t)tn * (BN / 2) + wn * (WTN / 2) + 32 * jj + c;
            ok = hcol < g.half_n;
            col = (j < TN / 2) ? hcol : g.half_n + hcol;
        } else {
            col = (int64_t)tn * BN + wn * WTN + 32 * j + c;
            ok = col < g.N;
        }
        vb_c[j] = ok ? (uint32_t)col * KB + 16u * hf : kOob;
        vb_s[j] = ok ? (uint32_t)col * KS : kOob;
    }

    auto load = [&](AFrag (&fa)[TM], Fp4Frag (&fb)[TN], int kc) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (AF == AFmt::kFp4) {
                fa[i].c = bload16(ra_c, va_c[i], (uint32_t)kc * 32u);
                fa[i].s = bload4(ra_s, va_s[i], (uint32_t)kc * 4u);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) fa[i].v[q] = bload16(ra_c, va_c[i] + 16u * q, (uint32_t)kc * 128u);
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            fb[j].c = bload16(rb_c, vb_c[j], (uint32_t)kc * 32u);
            fb[j].s = bload4(rb_s, vb_s[j], (uint32_t)kc * 4u);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto compute = [&](const AFrag (&fa)[TM], const Fp4Frag (&fb)[TN]) {
        f32x2 sa[TM], sb[TN];
        if constexpr (AF == AFmt::kFp4) {
#pragma unroll
            for (int i = 0; i < TM; ++i) sa[i] = frag_scales(fa[i].s, hf);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) sb[j] = frag_scales(fb[j].s, hf);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            Op av[TM], bv[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if constexpr (AF == AFmt::kFp4) {
                    av[i] = decode<Op>(word(fa[i].c, kk), kk < 2 ? sa[i].x : sa[i].y);
                } else {
                    av[i] = __builtin_bit_cast(Op, fa[i].v[kk]);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) bv[j] = decode<Op>(word(fb[j].c, kk), kk < 2 ? sb[j].x : sb[j].y);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma(av[i], bv[j], acc[i][j]);
        }
    };

    // Two register sets used in turn: the loads of step s + 1 are in flight
    // while step s is decoded and multiplied.
    AFrag fa0[TM], fa1[TM];
    Fp4Frag fb0[TN], fb1[TN];
    // (The scheduling barriers keep each step's loads ahead of the previous
    // step's MFMAs; left alone, the scheduler sinks them to shorten live
    // ranges, which exposes the load latency.)
    if (nsteps > 0) load(fa0, fb0, kc0);
    for (int s = 0; s + 1 < nsteps; s += 2) {
        load(fa1, fb1, kc0 + s + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(fa0, fb0);
        // Unconditional (the last pair re-reads its final step): a load under
        // a branch would make the next wait drain every load in flight.
        load(fa0, fb0, kc0 + min(s + 2, nsteps - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(fa1, fb1);
    }
    if (nsteps & 1) compute(fa0, fb0);

    // ---- epilogue: lane holds rows 8 (r/4) + 4 hf + r%4 of each 32x32 block, column c
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
                    const int64_t hcol = (int64_t)tn * (BN / 2) + wn * (WTN / 2) + 32 * j + c;
                    if (hcol >= g.half_n) continue;
                    const float gv = acc[i][j][r] * sc;
                    const float uv = acc[i][j + TN / 2][r] * sc;
                    const float hv = gv / (1.0f + expf(-gv)) * uv;
                    reinterpret_cast<uint16_t*>(g.out)[row * g.ldo + hcol] = (uint16_t)f32_to_bf16_rne(hv);
                }
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t col = (int64_t)tn * BN + wn * WTN + 32 * j + c;
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

template <int TM, int TN, int WM, int WN, AFmt AF, Epi EP>
hipError_t launch_cfg(const GemmArgs& g, int grid_m, hipStream_t stream) {
    constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
    dim3 grid;
    if (g.groups > 0) {
        const int64_t ncols = (EP == Epi::kMoeGateUp) ? g.half_n : g.N;
        const int64_t bn = (EP == Epi::kMoeGateUp) ? BN / 2 : BN;
        grid = dim3((unsigned)((ncols + bn - 1) / bn), (unsigned)grid_m, (unsigned)g.ksplit);
    } else {
        const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.ksplit;
        grid = dim3((unsigned)tiles);
    }
    hipLaunchKernelGGL((k_gemm_rd<TM, TN, WM, WN, AF, EP>), grid, dim3(64 * WM * WN), 0, stream, g);
    return hipGetLastError();
}

template <AFmt AF, Epi EP>
hipError_t launch_rd_tile(const GemmArgs& g, RdTile tile, int grid_m, hipStream_t stream) {
    switch (tile) {
        case RdTile::k128x128_w64x64: return launch_cfg<2, 2, 2, 2, AF, EP>(g, grid_m, stream);
        case RdTile::k256x128_w128x64: return launch_cfg<4, 2, 2, 2, AF, EP>(g, grid_m, stream);
        case RdTile::k128x256_w64x128: return launch_cfg<2, 4, 2, 2, AF, EP>(g, grid_m, stream);
        case RdTile::k256x256_w128x128: return launch_cfg<4, 4, 2, 2, AF, EP>(g, grid_m, stream);
        case RdTile::k128x256_w128x64: return launch_cfg<4, 2, 1, 4, AF, EP>(g, grid_m, stream);
        default: break;
    }
    if constexpr (EP != Epi::kMoeGateUp) {  // one column block per wave: no gate/up pairing
        switch (tile) {
            case RdTile::k128x128_w128x32: return launch_cfg<4, 1, 1, 4, AF, EP>(g, grid_m, stream);
            case RdTile::k64x128_w64x32: return launch_cfg<2, 1, 1, 4, AF, EP>(g, grid_m, stream);
            case RdTile::k32x128_w32x32: return launch_cfg<1, 1, 1, 4, AF, EP>(g, grid_m, stream);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

int rd_tile_rows(RdTile t) {
    switch (t) {
        case RdTile::k128x128_w64x64: return 128;
        case RdTile::k256x128_w128x64: return 256;
        case RdTile::k128x256_w64x128: return 128;
        case RdTile::k256x256_w128x128: return 256;
        case RdTile::k128x128_w128x32: return 128;
        case RdTile::k128x256_w128x64: return 128;
        case RdTile::k64x128_w64x32: return 64;
        case RdTile::k32x128_w32x32: return 32;
    }
    return 0;
}

int rd_tile_cols(RdTile t) {
    switch (t) {
        case RdTile::k128x128_w64x64: return 128;
        case RdTile::k256x128_w128x64: return 128;
        case RdTile::k128x256_w64x128: return 256;
        case RdTile::k256x256_w128x128: return 256;
        case RdTile::k128x128_w128x32: return 128;
        case RdTile::k128x256_w128x64: return 256;
        case RdTile::k64x128_w64x32: return 128;
        case RdTile::k32x128_w32x32: return 128;
    }
    return 0;
}

hipError_t launch_gemm_rd(const GemmArgs& g, AFmt afmt, Epi epi, RdTile tile, int grid_m,
                          hipStream_t stream) {
#define NVFP4_EPI(AF)                                                                        \
    switch (epi) {                                                                           \
        case Epi::kStoreBf16: return launch_rd_tile<AF, Epi::kStoreBf16>(g, tile, grid_m, stream);   \
        case Epi::kPartialF32: return launch_rd_tile<AF, Epi::kPartialF32>(g, tile, grid_m, stream); \
        case Epi::kMoeGateUp: return launch_rd_tile<AF, Epi::kMoeGateUp>(g, tile, grid_m, stream);   \
        case Epi::kMoeDown: return launch_rd_tile<AF, Epi::kMoeDown>(g, tile, grid_m, stream);       \
    }
    switch (afmt) {
        case AFmt::kFp4: NVFP4_EPI(AFmt::kFp4) break;
        case AFmt::kF16: NVFP4_EPI(AFmt::kF16) break;
        case AFmt::kBf16: NVFP4_EPI(AFmt::kBf16) break;
    }
#undef NVFP4_EPI
    return hipErrorInvalidValue;
}

}  // namespace nvfp4
