// gemm_a16.hip -- NVFP4-weight GEMM with a 16-bit activation operand:
// Y = A * W^T, A [M, K] f16 (the exact values q * s of an NVFP4-quantized
// activation: the W4A4 path) or bf16 (the W4A16 path), W NVFP4 [N, K].
//
// Fprop with the contraction axis innermost on both operands ("Getting
// GLM-5.2 NVFP4 Post-Training off the ground", "Going deeper" and "TN, NT,
// and what actually binds"); W4A4 and W4A16 per the model card
// "vroomfondel/glm-5.2-reap-504B-v2-W4A4", "Kernel choice".
//
// Scale application: weight elements are decoded to q * s, exact in f16 and
// in bf16, and multiplied on v_mfma_f32_32x32x16_{f16,bf16} with fp32
// accumulation; the global scales are applied in the epilogue.  gfx950's
// scaled MFMA takes one power-of-two scale per 32 elements and its fp4
// conversions use only the exponent of their scale operand, so neither can
// carry a per-16 E4M3 scale; decoding costs VALU work, which is why the
// activation arrives already decoded (its quantizer writes q * s directly)
// and only the weight tile is decoded here, once per wave that uses it.
//
// Data movement, per 64-wide K step (double-buffered in LDS, one barrier per
// step): the workgroup loads the A tile (BM rows x 128 bytes, 8 lanes per
// row) and the packed B tile (BN rows x 32 code bytes + 4 scale bytes)
// through registers into LDS.  Waves read A fragments and packed B fragments
// from LDS, decode B in registers and issue the MFMAs.
//
// K order inside a step: the 32x32x16 MFMA takes, in lane l, row (or column)
// l % 32 and 8 consecutive K positions selected by l / 32.  A K permutation
// applied to both operands leaves the product unchanged, so lane half
// hf = l / 32 takes K positions [32 hf, 32 hf + 32) of the step and MFMA kk
// uses positions 32 hf + 8 kk + [0, 8): a lane's packed B share is 16
// contiguous code bytes and two scale bytes.
//
// LDS rows are padded (A: 144 bytes, B codes: 48 bytes) so that the 16-byte
// reads of 16 consecutive rows fall on distinct banks.
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
__device__ __forceinline__ uint32_t bload4(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <AFmt AF>
struct OpOf;
template <>
struct OpOf<AFmt::kF16> {
    using T = f16x8;
};
template <>
struct OpOf<AFmt::kBf16> {
    using T = bf16x8;
};

// Eight weight codes (one word) -> eight operand values q * s (exact).
__device__ __forceinline__ f16x8 decode_w(uint32_t w, float s, f16x8*) {
    return fp4x8_scaled_f16(w, (_Float16)s);
}
__device__ __forceinline__ bf16x8 decode_w(uint32_t w, float s, bf16x8*) {
    return __builtin_bit_cast(bf16x8, fp4x8_scaled_bf16_bits(w, s));
}

__device__ __forceinline__ uint32_t word(const uint4& v, int kk) {
    return kk == 0 ? v.x : kk == 1 ? v.y : kk == 2 ? v.z : v.w;
}

constexpr int kRowA = 144;   // LDS bytes per A row per step (128 + 16 of padding)
constexpr int kRowB = 48;    // LDS bytes per B row of codes per step (32 + 16 of padding)
constexpr int kGroupM = 8;   // m-tiles per band in the ungrouped tile order

template <int TM, int TN, int WM, int WN>
struct Cfg {
    static constexpr int NW = WM * WN, NT = 64 * NW;
    static constexpr int WTM = 32 * TM, WTN = 32 * TN;
    static constexpr int BM = WTM * WM, BN = WTN * WN;
    static constexpr int A_BYTES = BM * kRowA, BC_BYTES = BN * kRowB, BS_BYTES = BN * 4;
    static constexpr int STAGE = A_BYTES + BC_BYTES + BS_BYTES;
    // per-thread share of one step's copy
    static constexpr int A_CHUNKS = BM * 8;                // 16-byte chunks of A
    static constexpr int A_PER_T = A_CHUNKS / NT;
    static constexpr int B_CHUNKS = BN * 2;                // 16-byte chunks of B codes
    static constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
    static_assert(A_CHUNKS % NT == 0, "A copy");
    static_assert(BN <= NT, "one scale word per thread");
    static_assert(2 * STAGE <= 160 * 1024, "LDS");
};

// WPE: minimum waves per SIMD the register allocation must allow (1: no
// constraint beyond the workgroup size).
template <int TM, int TN, int WM, int WN, int PD, AFmt AF, Epi EP, int WPE>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE)))
void k_gemm_a16(GemmArgs g) {
    using C = Cfg<TM, TN, WM, WN>;
    using Op = typename OpOf<AF>::T;
    constexpr int BM = C::BM, BN = C::BN, WTM = C::WTM, WTN = C::WTN;
    constexpr bool kGateUp = EP == Epi::kMoeGateUp || EP == Epi::kMoeGateUpLora;
    constexpr bool kLora = EP == Epi::kMoeGateUpLora || EP == Epi::kMoeDownLora;
    static_assert(!kGateUp || (TN % 2) == 0, "gate/up needs paired column blocks");
    __shared__ __align__(16) uint8_t smem[2 * C::STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int c32 = lane & 31, hf = lane >> 5;

    // ---- tile, group and K range of this workgroup.  Workgroups are dealt to
    // the 8 XCDs round-robin by linear id; the id is renumbered so that each
    // XCD receives a contiguous run of the real tiles (a grouped launch is
    // sized for the worst case: its surplus workgroups hold ids past the real
    // tile count, read from tile_off on the device, and exit).  Grouped
    // problems walk the column tiles of one row tile consecutively (they share
    // the row tile's activations in that XCD's L2); ungrouped ones walk bands
    // of kGroupM row tiles so that concurrent tiles share both operands.
    const int nwg = (int)gridDim.x;
    const int gm_tiles = g.groups > 0 ? g.tile_off[g.groups] : 0;
    const int total = g.groups > 0 ? gm_tiles * g.grouped_ntiles * g.ksplit : nwg;
    int id = (int)blockIdx.x;
    if ((nwg & 7) == 0) {
        const int per_xcd = (total + 7) >> 3, j = id >> 3;
        if (j >= per_xcd) return;
        id = (id & 7) * per_xcd + j;
    }
    if (id >= total) return;
    int grp = 0, tn, kz;
    int64_t row_beg, row_end;
    if (g.groups > 0) {
        const int ntiles = g.grouped_ntiles;
        kz = id / (ntiles * gm_tiles);
        const int t = id - kz * ntiles * gm_tiles;
        const int mt = t / ntiles;
        tn = t - mt * ntiles;
        int lo = 0, hi = g.groups;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (g.tile_off[mid] <= mt) lo = mid; else hi = mid;
        }
        grp = lo;
        row_beg = (int64_t)g.row_off[grp] + (int64_t)(mt - g.tile_off[grp]) * BM;
        row_end = min((int64_t)g.row_off[grp + 1], row_beg + BM);
    } else {
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
    const int ksteps = (int)(g.K / 64);
    const int per = (ksteps + g.ksplit - 1) / g.ksplit;
    const int kc0 = __builtin_amdgcn_readfirstlane(kz * per);
    int nsteps = __builtin_amdgcn_readfirstlane(max(0, min(ksteps - kc0, per)));
    const int gi = g.groups > 0 ? grp : 0;
    float sc = (g.a_global ? g.a_global[gi] : 1.0f) * (g.b_global ? g.b_global[gi] : 1.0f);
    // LoRA overlay: the accumulators start at (lora_scale / sc) * (Z Bg^T),
    // so that the epilogue's sc * acc adds lora_scale * (Z Bg^T) to the
    // weight product.  If that ratio is not finite (sc is zero or nearly),
    // the weight product vanishes: the K loop is skipped and the epilogue
    // multiplies Z Bg^T by lora_scale alone.
    float lora_mul = 0.0f;
    if constexpr (kLora) {
        const float ratio = g.lora_scale / sc;
        if (fabsf(ratio) <= 3.402823466e38f) {
            lora_mul = ratio;
        } else {
            nsteps = 0;
            lora_mul = 1.0f;
            sc = g.lora_scale;
        }
    }

    const uint32_t KB = (uint32_t)(g.K / 2), KS = (uint32_t)(g.K / 16), KA = (uint32_t)(g.K * 2);
    // A: 16-bit rows, optionally gathered, one resource over the source tensor
    // (the host keeps it below 2 GiB)
    const Rsrc ra = make_rsrc(g.a, (uint64_t)g.a_src_rows * KA);
    const Rsrc rb_c = make_rsrc(g.b_codes + (int64_t)grp * g.N * KB, (uint64_t)g.N * KB);
    const Rsrc rb_s = make_rsrc(g.b_scales + (int64_t)grp * g.N * KS, (uint64_t)g.N * KS);

    // Global column of tile column n (or -1 past the end).
    auto b_col = [&](int n) -> int64_t {
        if constexpr (kGateUp) {
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
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // LoRA overlay (see lora_mul): one bf16 contraction of length R per 32x32
    // block, Z rows against the group's B rows (the output columns of the
    // weight rows of this tile, gate/up order included), read straight from
    // global memory in the MFMA operand layout, 64 ranks at a time with the
    // loads of all blocks in flight together.  It runs before the K loop's
    // address set-up and first loads, while few registers are live; the other
    // workgroups on the CU cover its one round trip to L2.
    if constexpr (kLora) {
        const int R = g.lora_rank;
        const uint16_t* bg = g.lora_b + (int64_t)grp * g.N * R;
        const uint16_t* bp[TN];
        const uint16_t* zp[TM];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = b_col(wn * WTN + 32 * j + c32);
            bp[j] = col >= 0 ? bg + col * R + 8 * hf : nullptr;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t row = row_beg + wm * WTM + 32 * i + c32;
            zp[i] = nullptr;
            if (row < row_end)
                zp[i] = g.lora_z + (int64_t)(g.lora_rows ? g.lora_rows[row] / g.lora_div : (int32_t)row) * R + 8 * hf;
        }
        for (int q0 = 0; q0 < R; q0 += 64) {   // uniform trip count
            u32x4 za[TM][4], zb[TN][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = q0 + 16 * u;
                const bool in = q + 8 * hf < R;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    za[i][u] = u32x4{0, 0, 0, 0};
                    if (zp[i] && in) za[i][u] = *reinterpret_cast<const u32x4*>(zp[i] + q);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    zb[j][u] = u32x4{0, 0, 0, 0};
                    if (bp[j] && in) zb[j][u] = *reinterpret_cast<const u32x4*>(bp[j] + q);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = mfma(__builtin_bit_cast(bf16x8, za[i][u]), __builtin_bit_cast(bf16x8, zb[j][u]),
                                         acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] *= lora_mul;
    }
    // ---- this thread's copy assignments (fixed for the whole K loop)
    // A: chunk p = tid + NT * u -> row p / 8, 16-byte chunk p % 8 of the row's step
    // LDS offsets are one per-thread base plus compile-time steps, so that
    // they cost one register each and the steps go into the instructions'
    // offset fields.
    uint32_t va[C::A_PER_T];
    const uint32_t la0 = (uint32_t)((tid >> 3) * kRowA + 16 * (tid & 7));
#pragma unroll
    for (int u = 0; u < C::A_PER_T; ++u) {
        const int p = tid + C::NT * u, r = p >> 3, cc = p & 7;
        const int64_t row = row_beg + r;
        uint32_t v = kOob;
        if (row < row_end) {
            const int64_t src = g.a_rows ? (int64_t)(g.a_rows[row] / g.a_div) : row;
            v = (uint32_t)(src * KA) + 16u * cc;
        }
        va[u] = v;
    }
    // B codes: chunk p = tid + NT * u (p < 2 BN) -> column p / 2, half p % 2
    uint32_t vbc[C::B_PER_T], lbc[C::B_PER_T];
#pragma unroll
    for (int u = 0; u < C::B_PER_T; ++u) {
        const int p = tid + C::NT * u;
        const int n = p >> 1, h2 = p & 1;
        uint32_t v = kOob;
        if (p < C::B_CHUNKS) {
            const int64_t col = b_col(n);
            if (col >= 0) v = (uint32_t)col * KB + 16u * h2;
        }
        vbc[u] = v;
        lbc[u] = C::A_BYTES + (p < C::B_CHUNKS ? n * kRowB + 16 * h2 : 0);
    }
    // B scales: thread tid < BN copies column tid's 4 scale bytes of the step
    uint32_t vbs = kOob;
    if (tid < BN) {
        const int64_t col = b_col(tid);
        if (col >= 0) vbs = (uint32_t)col * KS;
    }
    const uint32_t lbs = C::A_BYTES + C::BC_BYTES + 4 * (tid < BN ? tid : 0);

    // PD register sets, each holding one step's share of the copy: step t
    // lives in set t % PD, so the loads of PD steps are in flight at once.
    struct StageRegs {
        uint4 a[C::A_PER_T], b[C::B_PER_T];
        uint32_t s;
    };
    StageRegs stg[PD];
    auto load_step = [&](StageRegs& r, int kc) {
#pragma unroll
        for (int u = 0; u < C::A_PER_T; ++u) r.a[u] = bload16(ra, va[u], (uint32_t)kc * 128u);
#pragma unroll
        for (int u = 0; u < C::B_PER_T; ++u) r.b[u] = bload16(rb_c, vbc[u], (uint32_t)kc * 32u);
        r.s = bload4(rb_s, vbs, (uint32_t)kc * 4u);
    };
    auto store_step = [&](const StageRegs& r, int buf) {
        uint8_t* base = smem + buf * C::STAGE;
#pragma unroll
        for (int u = 0; u < C::A_PER_T; ++u) *reinterpret_cast<uint4*>(base + la0 + u * (C::NT / 8) * kRowA) = r.a[u];
#pragma unroll
        for (int u = 0; u < C::B_PER_T; ++u)
            if (tid + C::NT * u < C::B_CHUNKS) *reinterpret_cast<uint4*>(base + lbc[u]) = r.b[u];
        if (tid < BN) *reinterpret_cast<uint32_t*>(base + lbs) = r.s;
    };

    // ---- fragment addresses within a stage buffer
    const uint32_t fa0 = (uint32_t)((wm * WTM + c32) * kRowA + 64 * hf);
    const uint32_t fbc0 = (uint32_t)(C::A_BYTES + (wn * WTN + c32) * kRowB + 16 * hf);
    const uint32_t fbs0 = (uint32_t)(C::A_BYTES + C::BC_BYTES + 4 * (wn * WTN + c32));
    auto fa = [&](int i) { return fa0 + 32 * i * kRowA; };
    auto fbc = [&](int j) { return fbc0 + 32 * j * kRowB; };
    auto fbs = [&](int j) { return fbs0 + 128 * j; };

    // One K step from LDS buffer `buf`: the A fragments of MFMA group kk + 1
    // are requested before the MFMAs of group kk are issued (the scheduling
    // barriers keep that order; left alone, the scheduler re-reads fragments
    // just in time to save registers and the MFMAs wait on LDS latency).
    // Waves whose rows all lie past the end of the row tile (a group's last,
    // partly filled tile) skip their MFMAs; the copy work stays shared.
    const bool wave_rows = (int64_t)wm * WTM < row_end - row_beg;
    auto compute_step = [&](int buf) {
        if (!wave_rows) return;
        const uint8_t* base = smem + buf * C::STAGE;
        uint4 cb[TN];
        f32x2 sb[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            cb[j] = *reinterpret_cast<const uint4*>(base + fbc(j));
            sb[j] = e4m3x2_to_f32(*reinterpret_cast<const uint32_t*>(base + fbs(j)) >> (16 * hf));
        }
        Op av[2][TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) av[0][i] = *reinterpret_cast<const Op*>(base + fa(i));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk + 1 < 4) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    av[(kk + 1) & 1][i] = *reinterpret_cast<const Op*>(base + fa(i) + 16 * (kk + 1));
            }
            Op bv[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bv[j] = decode_w(word(cb[j], kk), kk < 2 ? sb[j].x : sb[j].y, (Op*)nullptr);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma(av[kk & 1][i], bv[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- main loop, one barrier per step: iteration s multiplies LDS buffer
    // s % 2, then writes step s + 1 from its register set into the other
    // buffer (last read in iteration s - 1, before the previous barrier) and
    // refills that set with step s + 1 + PD.  Loads past the last step re-read
    // it (the clamp keeps the load count per iteration fixed, so the waits
    // stay exact); their data is never multiplied.
    if (nsteps > 0) {
#pragma unroll
        for (int u = 0; u < PD; ++u) load_step(stg[u], kc0 + min(u, nsteps - 1));
        store_step(stg[0], 0);
        load_step(stg[0], kc0 + min(PD, nsteps - 1));
        __syncthreads();
    }
    auto step = [&](int s, StageRegs& next) {
        compute_step(s & 1);
        store_step(next, (s + 1) & 1);
        load_step(next, kc0 + min(s + 1 + PD, nsteps - 1));
        __syncthreads();
    };
    // whole groups of PD steps without conditions (exact wait counts), then
    // the remaining steps
    const int nmain = nsteps / PD * PD;
    for (int s0 = 0; s0 < nmain; s0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) step(s0 + u, stg[(u + 1) % PD]);
    }
#pragma unroll
    for (int u = 0; u < PD; ++u)
        if (nmain + u < nsteps) step(nmain + u, stg[(u + 1) % PD]);

    // ---- epilogue: lane holds rows 8 (r/4) + 4 hf + r%4 of each 32x32 block, column c32
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = row_beg + wm * WTM + 32 * i + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (row >= row_end) continue;
            if constexpr (kGateUp) {
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

template <int TM, int TN, int WM, int WN, int PD, AFmt AF, Epi EP, int WPE = 1>
hipError_t launch_cfg(const GemmArgs& g0, int grid_m, hipStream_t stream) {
    using C = Cfg<TM, TN, WM, WN>;
    GemmArgs g = g0;
    int64_t wgs;
    if (g.groups > 0) {
        // grid_m bounds the row tiles of all groups; surplus workgroups exit
        constexpr bool kGateUp = EP == Epi::kMoeGateUp || EP == Epi::kMoeGateUpLora;
        const int64_t ncols = kGateUp ? g.half_n : g.N;
        const int64_t bn = kGateUp ? C::BN / 2 : C::BN;
        g.grouped_ntiles = (int32_t)((ncols + bn - 1) / bn);
        wgs = (int64_t)g.grouped_ntiles * grid_m * g.ksplit;
        wgs = (wgs + 7) / 8 * 8;  // a multiple of 8 for the XCD renumbering
    } else {
        wgs = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN) * g.ksplit;
    }
    hipLaunchKernelGGL((k_gemm_a16<TM, TN, WM, WN, PD, AF, EP, WPE>), dim3((unsigned)wgs), dim3(C::NT), 0, stream, g);
    return hipGetLastError();
}

template <AFmt AF, Epi EP>
hipError_t launch_tile(const GemmArgs& g, A16Tile tile, int grid_m, hipStream_t stream) {
    switch (tile) {
        case A16Tile::k256x256_w128x64: return launch_cfg<4, 2, 2, 4, 2, AF, EP>(g, grid_m, stream);
        case A16Tile::k256x256_w128x128: return launch_cfg<4, 4, 2, 2, 1, AF, EP>(g, grid_m, stream);
        case A16Tile::k256x128_w128x64: return launch_cfg<4, 2, 2, 2, 1, AF, EP>(g, grid_m, stream);
        case A16Tile::k256x128_w64x64: return launch_cfg<2, 2, 4, 2, 1, AF, EP>(g, grid_m, stream);
        case A16Tile::k128x256_w64x128: return launch_cfg<2, 4, 2, 2, 1, AF, EP>(g, grid_m, stream);
        case A16Tile::k128x128_w64x64: return launch_cfg<2, 2, 2, 2, 2, AF, EP, 3>(g, grid_m, stream);
        case A16Tile::k128x128_w32x64: return launch_cfg<1, 2, 4, 2, 2, AF, EP>(g, grid_m, stream);
        case A16Tile::k64x256_w64x64: return launch_cfg<2, 2, 1, 4, 4, AF, EP>(g, grid_m, stream);
        case A16Tile::k32x256_w32x64: return launch_cfg<1, 2, 1, 4, 4, AF, EP>(g, grid_m, stream);
    }
    return hipErrorInvalidValue;
}

// Split-K finish: y = bf16(scale * sum_s partial[s]) with the splits summed
// in order.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ partial, int ksplit,
                                                       int64_t M, int64_t N, const float* __restrict__ g0,
                                                       const float* __restrict__ g1, uint16_t* __restrict__ y) {
    const float scale = *g0 * (g1 ? *g1 : 1.0f);
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        float s = 0.0f;
        for (int k = 0; k < ksplit; ++k) s += partial[(int64_t)k * total + i];
        y[i] = (uint16_t)f32_to_bf16_rne(s * scale);
    }
}

}  // namespace

int a16_tile_rows(A16Tile t) {
    switch (t) {
        case A16Tile::k256x256_w128x64: return 256;
        case A16Tile::k256x256_w128x128: return 256;
        case A16Tile::k256x128_w128x64: return 256;
        case A16Tile::k256x128_w64x64: return 256;
        case A16Tile::k128x256_w64x128: return 128;
        case A16Tile::k128x128_w64x64: return 128;
        case A16Tile::k128x128_w32x64: return 128;
        case A16Tile::k64x256_w64x64: return 64;
        case A16Tile::k32x256_w32x64: return 32;
    }
    return 0;
}

int a16_tile_cols(A16Tile t) {
    switch (t) {
        case A16Tile::k256x256_w128x64: return 256;
        case A16Tile::k256x256_w128x128: return 256;
        case A16Tile::k256x128_w128x64: return 128;
        case A16Tile::k256x128_w64x64: return 128;
        case A16Tile::k128x256_w64x128: return 256;
        case A16Tile::k128x128_w64x64: return 128;
        case A16Tile::k128x128_w32x64: return 128;
        case A16Tile::k64x256_w64x64: return 256;
        case A16Tile::k32x256_w32x64: return 256;
    }
    return 0;
}

hipError_t launch_gemm_a16(const GemmArgs& g, AFmt afmt, Epi epi, A16Tile tile, int grid_m,
                           hipStream_t stream) {
#define NVFP4_EPI(AF)                                                                     \
    switch (epi) {                                                                        \
        case Epi::kStoreBf16: return launch_tile<AF, Epi::kStoreBf16>(g, tile, grid_m, stream);   \
        case Epi::kPartialF32: return launch_tile<AF, Epi::kPartialF32>(g, tile, grid_m, stream); \
        case Epi::kMoeGateUp: return launch_tile<AF, Epi::kMoeGateUp>(g, tile, grid_m, stream);   \
        case Epi::kMoeDown: return launch_tile<AF, Epi::kMoeDown>(g, tile, grid_m, stream);       \
        case Epi::kMoeGateUpLora:                                                         \
            if (tile != A16Tile::k128x128_w64x64) break;                                  \
            return launch_cfg<2, 2, 2, 2, 2, AF, Epi::kMoeGateUpLora, 3>(g, grid_m, stream); \
        case Epi::kMoeDownLora:                                                           \
            if (tile != A16Tile::k128x128_w64x64) break;                                  \
            return launch_cfg<2, 2, 2, 2, 2, AF, Epi::kMoeDownLora, 3>(g, grid_m, stream);   \
    }
    switch (afmt) {
        case AFmt::kF16: NVFP4_EPI(AFmt::kF16) break;
        case AFmt::kBf16: NVFP4_EPI(AFmt::kBf16) break;
        default: break;
    }
#undef NVFP4_EPI
    return hipErrorInvalidValue;
}

hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int64_t N,
                                const float* g0, const float* g1, uint16_t* y, hipStream_t stream) {
    int64_t grid = (M * N + 255) / 256;
    if (grid > 8192) grid = 8192;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)grid), dim3(256), 0, stream, partial, ksplit, M, N, g0, g1,
                       y);
    return hipGetLastError();
}

}  // namespace nvfp4
