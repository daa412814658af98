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
// Data movement, per 64-wide K step: the A tile (BM rows x 128 bytes) and the
// packed B tile (BN rows x 32 code bytes + 4 scale bytes) go from global
// memory straight into LDS (buffer_load ... lds: each load instruction of a
// wave fills 1 KB of LDS, 16 bytes per lane in lane order, or 256 bytes with
// 4-byte loads), into one of NS stage buffers, so that NS - 1 steps are in
// flight while a step is multiplied; one barrier per step.  Waves read A
// fragments and packed B fragments from LDS, decode B in registers and issue
// the MFMAs.
//
// K order inside a step: the 32x32x16 MFMA takes, in lane l, row (or column)
// l % 32 and 8 consecutive K positions selected by l / 32.  A K permutation
// applied to both operands leaves the product unchanged, so lane half
// hf = l / 32 takes K positions [32 hf, 32 hf + 32) of the step and MFMA kk
// uses positions 32 hf + 8 kk + [0, 8): a lane's packed B share is 16
// contiguous code bytes and two scale bytes.
//
// LDS rows are not padded (the copy fixes the layout); instead the 16-byte
// chunks of a row are permuted so that the 16-byte fragment reads of 16
// consecutive rows fall on distinct banks: A row r keeps its chunk c in slot
// c ^ ((r / 2) % 8), B column n its code half h in slot h ^ ((n / 8) % 2).
#include <algorithm>

#include "nvfp4_device.hpp"
#include "nvfp4_dma.hpp"
#include "nvfp4_encode.hpp"
#include "nvfp4_internal.hpp"

namespace nvfp4 {

namespace {

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

constexpr int kGroupM = 8;   // m-tiles per band in the ungrouped tile order

// Stream-K: workgroup w of W takes global K steps [floor(w S / W),
// floor((w + 1) S / W)); the one whose range holds step x.
__host__ __device__ __forceinline__ int sk_first(int64_t x, int W, int64_t S) {
    return (int)(((x + 1) * (int64_t)W - 1) / S);
}

// Tile geometry and the per-step copy.  The copy is cut into 1 KB slabs, one
// per 16-byte load instruction of a wave: 8 rows of A (128 bytes each), 32
// columns of B codes (32 bytes each); the scales take one 4-byte load per
// 64 columns.  With three or more stages every wave issues the same number
// of loads per step (waves without a B or scale slab load past the end of
// the buffer, which writes zeros to an unused slab), so that the vmcnt waits
// are exact; with two stages each step waits for all of its loads.
template <int TM, int TN, int WM, int WN, int NS>
struct Cfg {
    static constexpr int NW = WM * WN, NT = 64 * NW;
    static constexpr int WTM = 32 * TM, WTN = 32 * TN;
    static constexpr int BM = WTM * WM, BN = WTN * WN;
    static constexpr int A_SLABS = BM / 8, A_PER_W = A_SLABS / NW;
    static constexpr int B_SLABS = BN / 32, B_PER_W = (B_SLABS + NW - 1) / NW;
    static constexpr int S_SLABS = BN / 64;
    static constexpr int A_BYTES = BM * 128, B_BYTES = NW * B_PER_W * 1024, S_BYTES = NW * 256;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int LOADS = A_PER_W + B_PER_W + 1;   // load instructions per wave per step
    static_assert(A_SLABS % NW == 0, "A copy");
    static_assert(S_SLABS <= NW, "one scale load per wave");
    static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS");
    static_assert(LOADS * (NS - 2) <= 63, "vmcnt");
};

// NS: LDS stage buffers (NS - 1 steps in flight).  WPE: minimum waves per
// SIMD the register allocation must allow (1: no constraint beyond the
// workgroup size).  SJ: 16-byte scale chunks per column the workgroup may
// preload (0: none; else the launcher guarantees at most 4 SJ K steps per
// workgroup; see the preload below).
template <int TM, int TN, int WM, int WN, int NS, AFmt AF, Epi EP, int WPE, int SJ = 0, bool K2 = false,
          bool SK = false>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE)))
void k_gemm_a16(GemmArgs g) {
    using C = Cfg<TM, TN, WM, WN, NS>;
    using Op = typename OpOf<AF>::T;
    constexpr int BM = C::BM, BN = C::BN, WTM = C::WTM, WTN = C::WTN;
    constexpr bool kGateUp = EP == Epi::kMoeGateUp || EP == Epi::kMoeGateUpLora;
    constexpr bool kLora = EP == Epi::kMoeGateUpLora || EP == Epi::kMoeDownLora;
    static_assert(!kGateUp || (TN % 2) == 0, "gate/up needs paired column blocks");
    // K2: a stage holds two K steps: two A tiles, then the weight codes of
    // both steps, 64 bytes per column (16-byte slot s of column n holding
    // chunk s ^ ((n / 4) % 4)), loaded 16 columns per instruction
    static_assert(!K2 || SJ > 0, "two-step stages need the scale preload");
    constexpr int STG = K2 ? 2 * C::A_BYTES + C::BN * 64 : C::STAGE;
    constexpr int SP_OFF = NS * STG;
    static_assert(SJ == 0 || (SJ <= 16 && (SJ & (SJ - 1)) == 0), "scale chunks");
    static_assert(NS * STG + C::BN * SJ * 16 <= 160 * 1024, "LDS");
    __shared__ __align__(1024) uint8_t smem[NS * STG + C::BN * SJ * 16];

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
    const int ksteps = (int)(g.K / 64);
    // Stream-K (SK: ungrouped, sk_wgs > 0): the tiles' K steps, tile after tile,
    // are dealt out evenly, workgroup id taking global steps [sk0, sk1); it
    // runs one pass of the body below per tile its range touches and writes
    // that tile's part to partial slot id - sk_first(tile), or, when it holds
    // the whole tile, the finished bf16 tile to sk_y.
    int64_t sk0 = 0, sk1 = 0;
    if constexpr (SK) {
        const int64_t S = (int64_t)((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * ksteps;
        sk0 = (int64_t)id * S / g.sk_wgs;
        sk1 = (int64_t)(id + 1) * S / g.sk_wgs;
        if (sk0 >= sk1) return;   // (the host keeps sk_wgs <= S: never taken)
    }
    for (;;) {
    int grp = 0, tn, kz;
    int kc0_, nsteps_;
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
        const int per = (ksteps + g.ksplit - 1) / g.ksplit;
        kc0_ = kz * per;
        nsteps_ = max(0, min(ksteps - kc0_, per));
    } else {
        const int mtiles = (int)((g.M + BM - 1) / BM);
        const int ntiles = (int)((g.N + BN - 1) / BN);
        const int per_split = mtiles * ntiles;
        int t;
        if constexpr (SK) {
            t = (int)(sk0 / ksteps);
            kc0_ = (int)(sk0 - (int64_t)t * ksteps);
            nsteps_ = (int)min((int64_t)(ksteps - kc0_), sk1 - sk0);
            kz = id - sk_first((int64_t)t * ksteps, g.sk_wgs, (int64_t)per_split * ksteps);
        } else {
            kz = id / per_split;
            t = id - kz * per_split;
            const int per = (ksteps + g.ksplit - 1) / g.ksplit;
            kc0_ = kz * per;
            nsteps_ = max(0, min(ksteps - kc0_, per));
        }
        const int band = t / (kGroupM * ntiles);
        const int first_m = band * kGroupM;
        const int gsz = min(mtiles - first_m, kGroupM);
        const int r = t - band * kGroupM * ntiles;
        const int tm = first_m + r % gsz;
        tn = r / gsz;
        row_beg = (int64_t)tm * BM;
        row_end = min(g.M, row_beg + BM);
    }
    const int kc0 = __builtin_amdgcn_readfirstlane(kc0_);
    const int seg_steps = __builtin_amdgcn_readfirstlane(nsteps_);
    int nsteps = seg_steps;
    const bool sk_whole = SK && kc0 == 0 && seg_steps == ksteps;
    const int gi = g.groups > 0 ? grp : 0;
    // First row of the wave within the tile.  Grouped tiles of 96-row waves
    // (TM = 3) whose rows fit two 64-row halves (an expert of at most
    // 2 x 64 rows) give each wave row 64 of them, so that no wave decodes
    // the weights for a single 32-row block; tm_cap is then 2.
    constexpr bool kDynRows = TM == 3 && EP != Epi::kStoreBf16 && EP != Epi::kPartialF32;
    const bool half_rows = kDynRows && row_end - row_beg <= 64 * WM;
    const int wrow = half_rows ? wm * 64 : wm * WTM;
    const int tm_cap = half_rows ? 2 : TM;
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
    const u32x4 ra = make_rsrc(g.a, (uint64_t)g.a_src_rows * KA);
    const u32x4 rb_c = make_rsrc(g.b_codes + (int64_t)grp * g.N * KB, (uint64_t)g.N * KB);
    const u32x4 rb_s = make_rsrc(g.b_scales + (int64_t)grp * g.N * KS, (uint64_t)g.N * KS);

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
            const int64_t row = row_beg + wrow + 32 * i + c32;
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
    // ---- this lane's copy assignments (fixed for the whole K loop)
    // A slab sl = A_PER_W wave + u: rows 8 sl + lane / 8, LDS slot lane % 8,
    // which receives the row's 16-byte chunk slot ^ ((row / 2) % 8).
    const bool a_gather = g.a_rows != nullptr && (g.a_rows_on == nullptr || *g.a_rows_on != 0);
    uint32_t va[C::A_PER_W];
#pragma unroll
    for (int u = 0; u < C::A_PER_W; ++u) {
        const int r = 8 * (C::A_PER_W * wave + u) + (lane >> 3);
        const int cc = (lane & 7) ^ ((r >> 1) & 7);
        const int64_t row = row_beg + r;
        uint32_t v = kOob;
        if (row < row_end) {
            const int64_t src = a_gather ? (int64_t)(g.a_rows[row] / g.a_div) : row;
            v = (uint32_t)(src * KA) + 16u * cc;
        }
        va[u] = v;
    }
    // B code slab sb = B_PER_W wave + u: columns 32 sb + lane / 2, LDS half
    // lane % 2, which receives the column's code half (lane % 2) ^ ((n / 8) % 2).
    uint32_t vbc[C::B_PER_W];
#pragma unroll
    for (int u = 0; u < C::B_PER_W; ++u) {
        const int sb = C::B_PER_W * wave + u;
        const int n = 32 * sb + (lane >> 1);
        const int h2 = (lane & 1) ^ ((n >> 3) & 1);
        uint32_t v = kOob;
        if (sb < C::B_SLABS) {
            const int64_t col = b_col(n);
            if (col >= 0) v = (uint32_t)col * KB + 16u * h2;
        }
        vbc[u] = v;
    }
    // B scales: wave w < S_SLABS loads the step's 4 scale bytes of columns 64 w + lane
    uint32_t vbs = kOob;
    if (wave < C::S_SLABS) {
        const int64_t col = b_col(64 * wave + lane);
        if (col >= 0) vbs = (uint32_t)col * KS;
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(smem));
    // Scale preload (SJ > 0): a K step of a column has only 4 scale bytes, so
    // a per-step scale load touches one cache line per 4 bytes.  Instead the
    // workgroup's scales (at most 4 SJ steps) are loaded once, 16 bytes (four
    // steps) per lane: column n keeps its chunk j in slot j ^ ((n / 2) % SJ)
    // of SJ 16-byte slots.
    constexpr bool sp = SJ > 0;
    constexpr int sj = SJ;
    // Step kc of this workgroup's K range into stage buffer st.
    constexpr int B2_PER_W = C::BN / 16 / C::NW;
    static_assert(!K2 || (C::BN / 16) % C::NW == 0, "two-step code slabs");
    uint32_t vbc2[K2 ? B2_PER_W : 1];
    if constexpr (K2) {
#pragma unroll
        for (int u = 0; u < B2_PER_W; ++u) {
            const int n = 16 * (B2_PER_W * wave + u) + (lane >> 2);
            const int c = (lane & 3) ^ ((n >> 2) & 3);
            const int64_t col = b_col(n);
            vbc2[u] = col >= 0 ? (uint32_t)col * KB + 16u * c : kOob;
        }
    }
    // group kg (steps 2 kg, 2 kg + 1 of the range, clamped) into stage st
    auto issue2 = [&](int kg, int st) {
        const uint32_t b = lds0 + (uint32_t)(st * STG);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int kc = kc0 + min(2 * kg + g, nsteps - 1);
#pragma unroll
            for (int u = 0; u < C::A_PER_W; ++u)
                lds_load16(ra, va[u], (uint32_t)kc * 128u, b + (uint32_t)(g * C::A_BYTES + (C::A_PER_W * wave + u) * 1024));
        }
#pragma unroll
        for (int u = 0; u < B2_PER_W; ++u)
            lds_load16(rb_c, vbc2[u], (uint32_t)(kc0 + 2 * kg) * 32u, b + (uint32_t)(2 * C::A_BYTES + (B2_PER_W * wave + u) * 1024));
    };
    // With two stages every step waits for all of its loads, so a wave may
    // skip the A slabs that lie wholly past the tile's last row (their LDS
    // rows then hold stale data, which only padding rows multiply and which
    // the epilogue never stores).
    bool a_live[C::A_PER_W];
#pragma unroll
    for (int u = 0; u < C::A_PER_W; ++u)
        a_live[u] = NS > 2 || (int64_t)8 * (C::A_PER_W * wave + u) < row_end - row_beg;
    auto issue = [&](int kc, int st) {
        const uint32_t b = lds0 + (uint32_t)(st * C::STAGE);
#pragma unroll
        for (int u = 0; u < C::A_PER_W; ++u)
            if (a_live[u]) lds_load16(ra, va[u], (uint32_t)kc * 128u, b + (uint32_t)((C::A_PER_W * wave + u) * 1024));
#pragma unroll
        for (int u = 0; u < C::B_PER_W; ++u)
            lds_load16(rb_c, vbc[u], (uint32_t)kc * 32u, b + (uint32_t)(C::A_BYTES + (C::B_PER_W * wave + u) * 1024));
        if constexpr (!sp) lds_load4(rb_s, vbs, (uint32_t)kc * 4u, b + (uint32_t)(C::A_BYTES + C::B_BYTES + 256 * wave));
    };

    // ---- fragment addresses within a stage buffer.  A: row wm WTM + 32 i +
    // c32, chunk 4 hf + kk, in slot (4 hf + kk) ^ ((c32 / 2) % 8) (the row's
    // other terms are multiples of 32); B: column wn WTN + 32 j + c32, code
    // half hf in slot hf ^ ((c32 / 8) % 2); scales: 4 bytes per column.
    uint32_t fa_k[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        fa_k[kk] = (uint32_t)((wrow + c32) * 128 + 16 * ((4 * hf + kk) ^ ((c32 >> 1) & 7)));
    const uint32_t fbc0 = (uint32_t)(C::A_BYTES + (wn * WTN + c32) * 32 + 16 * (hf ^ ((c32 >> 3) & 1)));
    const uint32_t fbs0 = (uint32_t)(C::A_BYTES + C::B_BYTES + 4 * (wn * WTN + c32));
    auto fa = [&](int i, int kk) { return fa_k[kk] + 32 * 128 * i; };
    auto fbc = [&](int j) { return fbc0 + 32 * 32 * j; };
    auto fbs = [&](int j) { return fbs0 + 128 * j; };

    // One K step from stage buffer `st`: the A fragments of MFMA group kk + 1
    // are requested before the MFMAs of group kk are issued (the scheduling
    // barriers keep that order; left alone, the scheduler re-reads fragments
    // just in time to save registers and the MFMAs wait on LDS latency).
    // Waves whose rows all lie past the end of the row tile (a group's last,
    // partly filled tile) skip their MFMAs; the copy work stays shared.
    const bool wave_rows = (int64_t)wrow < row_end - row_beg;
    // Grouped tiles: a wave skips the MFMAs of its 32-row blocks that hold
    // only padding (wave_blocks: the blocks with at least one real row).
    constexpr bool kBlockSkip = (TM == 2 || TM == 3) && EP != Epi::kStoreBf16 && EP != Epi::kPartialF32;
    const int wave_blocks =
        kBlockSkip ? (int)min((int64_t)tm_cap, (row_end - row_beg - (int64_t)wrow + 31) / 32) : TM;
    const int gsc = (c32 >> 1) & (sj > 0 ? sj - 1 : 0);
    // (the tile's column offsets wn WTN + 32 j are multiples of 32, so the
    // slot permutation of column wn WTN + 32 j + c32 depends on c32 alone)
    const uint32_t fsp0 = (uint32_t)(SP_OFF + (wn * WTN + c32) * sj * 16);
    auto compute_at = [&](const uint8_t* base, const uint8_t* cbase, int cstride, int ls) {
        if (!wave_rows) return;
        uint4 cb[TN];
        f32x2 sb[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            cb[j] = *reinterpret_cast<const uint4*>(cbase + cstride * j);
            const uint8_t* sa = base + fbs(j);
            if constexpr (sp) sa = smem + fsp0 + 32 * j * sj * 16 + 16 * ((ls >> 2) ^ gsc) + 4 * (ls & 3);
            sb[j] = e4m3x2_to_f32(*reinterpret_cast<const uint32_t*>(sa) >> (16 * hf));
        }
        if constexpr (TM == 4) {
            // 128-row waves: a software pipeline.  The A reads and the weight
            // decode of group kk + 1 are issued among the MFMAs of group kk,
            // one MFMA then kVpm VALU instructions (the decode's VALU count
            // per MFMA of the group), so the single MFMA pipe of the SIMD is
            // fed while the wave decodes.  Each accumulator sees the same
            // MFMAs in the same order as without it.  Measured on MI355X
            // (dense M = 4096): W4A4 +5-10 %, W4A16 +11-15 %; the 64-row-wave
            // tiles did not gain and keep the plain order below.
            constexpr int kVpm = ((AF == AFmt::kBf16 ? 16 : 8) + TM - 1) / TM;
            Op av[2][TM], bv[2][TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) av[0][i] = *reinterpret_cast<const Op*>(base + fa(i, 0));
#pragma unroll
            for (int j = 0; j < TN; ++j) bv[0][j] = decode_w(word(cb[j], 0), sb[j].x, (Op*)nullptr);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int cur = kk & 1, nxt = cur ^ 1;
                if (kk + 1 < 4) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) av[nxt][i] = *reinterpret_cast<const Op*>(base + fa(i, kk + 1));
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        bv[nxt][j] = decode_w(word(cb[j], kk + 1), kk + 1 < 2 ? sb[j].x : sb[j].y, (Op*)nullptr);
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma(av[cur][i], bv[cur][j], acc[i][j]);
                if (kk + 1 < 4) {
                    __builtin_amdgcn_sched_group_barrier(0x100, TM, 0);       // the next group's A reads
#pragma unroll
                    for (int t = 0; t < TM * TN; ++t) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, kVpm, 0); // then VALU
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            Op av[2][TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) av[0][i] = *reinterpret_cast<const Op*>(base + fa(i, 0));
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk + 1 < 4) {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        av[(kk + 1) & 1][i] = *reinterpret_cast<const Op*>(base + fa(i, kk + 1));
                }
                Op bv[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bv[j] = decode_w(word(cb[j], kk), kk < 2 ? sb[j].x : sb[j].y, (Op*)nullptr);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if (i > 0 && i >= wave_blocks) break;
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma(av[kk & 1][i], bv[j], acc[i][j]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    auto compute_step = [&](int st, int ls) {
        const uint8_t* base = smem + st * C::STAGE;
        compute_at(base, base + fbc(0), 32 * 32, ls);
    };
    const uint32_t fbc2_0 = (uint32_t)(2 * C::A_BYTES + (wn * WTN + c32) * 64);
    auto compute_group = [&](int st, int kg) {
        const uint8_t* base = smem + st * STG;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int ls = 2 * kg + g;
            if (ls < nsteps)
                compute_at(base + g * C::A_BYTES, base + fbc2_0 + 16 * ((2 * g + hf) ^ ((c32 >> 2) & 3)), 32 * 64, ls);
        }
    };

    // ---- main loop, one barrier per step.  Iteration s issues step
    // s + NS - 1 into stage (s + NS - 1) % NS (multiplied in iteration s - 1,
    // before the previous barrier), multiplies stage s % NS, then waits until
    // step s + 1 has landed (only the loads of steps s + 2 .. s + NS - 1 may
    // remain) and meets the barrier.  Loads past the last step re-read it, so
    // every iteration issues C::LOADS loads per wave and the waits stay
    // exact; their data is never multiplied.
    // (with the scale preload a step issues one load fewer per wave)
    constexpr int kWaitNext = vmcnt_imm((sp ? C::LOADS - 1 : C::LOADS) * (NS - 2));
    auto wait_next = [&]() { __builtin_amdgcn_s_waitcnt(kWaitNext); };
    if constexpr (sp) {
        if (nsteps > 0) {
            // slot p = 64 u + lane holds column p / sj, chunk (p % sj) ^ ((n / 2) % sj);
            // chunks past the K range read the next scales of the row (or zeros
            // past the tensor) and are never used
            constexpr int ni = C::BN * sj / 64;
            for (int u = wave; u < ni; u += C::NW) {
                const int p = 64 * u + lane, n = p / sj, j = (p % sj) ^ ((n >> 1) & (sj - 1));
                const int64_t col = b_col(n);
                const uint32_t v = col >= 0 ? (uint32_t)col * KS + (uint32_t)kc0 * 4u + 16u * j : kOob;
                lds_load16(rb_s, v, 0u, lds0 + (uint32_t)(SP_OFF + 1024 * u));
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
    }
    if constexpr (K2) {
        constexpr int kWait2 = vmcnt_imm((2 * C::A_PER_W + B2_PER_W) * (NS - 2));
        const int ngroups = (nsteps + 1) / 2;
        if (nsteps > 0) {
#pragma unroll
            for (int u = 0; u + 1 < NS; ++u) issue2(min(u, ngroups - 1), u);
            __builtin_amdgcn_s_waitcnt(kWait2);
            __syncthreads();
        }
        auto gstep = [&](int s, int st) {
            issue2(min(s + NS - 1, ngroups - 1), (st + NS - 1) % NS);
            compute_group(st, s);
            __builtin_amdgcn_s_waitcnt(kWait2);
            __syncthreads();
        };
        const int gmain = ngroups / NS * NS;
        for (int s0 = 0; s0 < gmain; s0 += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u) gstep(s0 + u, u);
        }
#pragma unroll
        for (int u = 0; u + 1 < NS; ++u)
            if (gmain + u < ngroups) gstep(gmain + u, u);
        nsteps = 0;   // the single-step loop below has nothing left to do
    }
    if (nsteps > 0) {
#pragma unroll
        for (int u = 0; u + 1 < NS; ++u) issue(kc0 + min(u, nsteps - 1), u);
        wait_next();
        __syncthreads();
    }
    auto step = [&](int s, int st) {
        issue(kc0 + min(s + NS - 1, nsteps - 1), (st + NS - 1) % NS);
        compute_step(st, s);
        wait_next();
        __syncthreads();
    };
    // whole groups of NS steps (stage numbers known at compile time), then
    // the remaining steps
    const int nmain = nsteps / NS * NS;
    for (int s0 = 0; s0 < nmain; s0 += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) step(s0 + u, u);
    }
#pragma unroll
    for (int u = 0; u + 1 < NS; ++u)
        if (nmain + u < nsteps) step(nmain + u, u);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // (the last steps' clamped re-reads may still be landing in the stage
    // buffers of other waves: the bf16 epilogue below reuses them only after
    // every wave has seen its own loads complete)
    if constexpr (EP == Epi::kStoreBf16 || EP == Epi::kPartialF32) __syncthreads();

    // ---- epilogue: lane holds rows 8 (r/4) + 4 hf + r%4 of each 32x32 block, column c32.
    // Gate/up with out_q also quantizes h to NVFP4 under q_global[group]:
    // the 16 lanes of a DPP row (lane / 16 fixed) hold the 16 consecutive
    // columns of one block of one row, so the block maximum is a 16-lane
    // reduction, and each lane encodes its own element with the quantizer's
    // rule (nvfp4_encode.hpp) and stores the exact product q * s as f16.
    // Whole bf16 tiles leave through LDS: each wave writes a 32-row slab of
    // its results there (the K loop ended on a barrier, so the stage buffers
    // are free) and reads it back as 16-byte pieces of rows, so that a store
    // instruction covers eight whole 128-byte row segments instead of two
    // half segments of 2-byte elements.  Ragged edges and row strides that
    // are not a multiple of 8 store element by element.
    constexpr bool kBf16Tile = EP == Epi::kStoreBf16 || EP == Epi::kPartialF32;
    constexpr int kSlab = TN * 64;   // bytes per row of a wave's 32-row slab
    static_assert(!kBf16Tile || C::NW * 32 * kSlab <= NS * STG, "epilogue slabs");
    if (kBf16Tile && (EP == Epi::kStoreBf16 || sk_whole)) {
        uint16_t* const yb = EP == Epi::kStoreBf16 ? reinterpret_cast<uint16_t*>(g.out) : g.sk_y;
        uint8_t* const slab = smem + wave * 32 * kSlab;
        const bool vec = (g.ldo & 7) == 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 8 * (r >> 2) + 4 * hf + (r & 3);
                    *reinterpret_cast<uint16_t*>(slab + rr * kSlab + (32 * j + c32) * 2) =
                        (uint16_t)f32_to_bf16_rne(acc[i][j][r] * sc);
                }
#pragma unroll 1
            for (int p = 0; p < 32 * kSlab / 1024; ++p) {
                const int e = 64 * p + lane, rr = e / (kSlab / 16), ch = e % (kSlab / 16);
                const uint4 v = *reinterpret_cast<const uint4*>(slab + rr * kSlab + 16 * ch);
                const int64_t row = row_beg + wrow + 32 * i + rr;
                const int64_t col = (int64_t)tn * BN + wn * WTN + 8 * ch;
                if (row >= row_end || col >= g.N) continue;
                uint16_t* const dst = yb + row * g.ldo + col;
                if (vec && col + 8 <= g.N) {
                    *reinterpret_cast<uint4*>(dst) = v;
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (col + q < g.N) dst[q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
                }
            }
        }
    } else {
    float sgq = 0.0f;
    if constexpr (kGateUp) {
        if (g.out_q) sgq = g.q_global[gi];
    }
    const float tq = 6.0f * sgq;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (i >= tm_cap) break;   // (64-row halves: the third block is the next wave's)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = row_beg + wrow + 32 * i + 8 * (r >> 2) + 4 * hf + (r & 3);
            // (the row depends on the lane only through hf, so the 16-lane
            // groups of the gate/up quantization below stay whole)
            if (row >= row_end) continue;
            if constexpr (kGateUp) {
#pragma unroll
                for (int j = 0; j < TN / 2; ++j) {
                    // half_n is a multiple of 64, so a 16-column block is wholly in or out
                    const int64_t hcol = (int64_t)tn * (BN / 2) + wn * (WTN / 2) + 32 * j + c32;
                    const bool ok = hcol < g.half_n;
                    const float gv = acc[i][j][r] * sc;
                    const float uv = acc[i][j + TN / 2][r] * sc;
                    const float hv = gv / (1.0f + expf(-gv)) * uv;
                    const uint32_t hb = f32_to_bf16_rne(hv);
                    if (g.out != nullptr && ok) reinterpret_cast<uint16_t*>(g.out)[row * g.ldo + hcol] = (uint16_t)hb;
                    if (g.out_q != nullptr) {
                        const BlockEnc be = block_enc(row16_max_u32(hb & 0x7FFFu), sgq, tq);
                        const uint32_t code = encode_one(hb, be);
                        const f16x2 qv = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 0);
                        const _Float16 v = qv.x * (_Float16)be.s;
                        if (ok) g.out_q[row * g.ldo + hcol] = __builtin_bit_cast(uint16_t, v);
                    }
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
                        if (sk_whole)
                            g.sk_y[row * g.ldo + col] = (uint16_t)f32_to_bf16_rne(v * sc);
                        else
                            reinterpret_cast<float*>(g.out)[((int64_t)kz * g.M + row) * g.ldo + col] = v;
                    } else {
                        reinterpret_cast<float*>(g.out)[row * g.ldo + col] = v * sc;
                    }
                }
            }
        }
    }
    }
    // next stream-K segment (the K loop ended on a barrier, so the stage
    // buffers are free once every wave has left its epilogue)
    if constexpr (!SK) {
        break;
    } else {
        sk0 += seg_steps;
        if (sk0 >= sk1) break;
        __syncthreads();   // the epilogue slabs share LDS with the next segment's stages
    }
    }
}

template <int TM, int TN, int WM, int WN, int NS, AFmt AF, Epi EP, int WPE = 1, int SJ = 0, bool K2 = false>
hipError_t launch_cfg(const GemmArgs& g0, int grid_m, hipStream_t stream) {
    using C = Cfg<TM, TN, WM, WN, NS>;
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
    } else if (g.sk_wgs > 0) {
        // stream-K: ungrouped partial sums with the per-step scale loads only
        // (the scale preload and the two-step stages assume one K range per
        // workgroup); built for the 256 x 256 tile, the one the plans use it on
        const int64_t steps = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN) * (g.K / 64);
        if constexpr (EP == Epi::kPartialF32 && SJ == 0 && !K2 && C::BM == 256 && C::BN == 256) {
            if (g.ksplit != 1 || g.sk_wgs > steps || g.sk_y == nullptr) return hipErrorInvalidValue;
            hipLaunchKernelGGL((k_gemm_a16<TM, TN, WM, WN, NS, AF, EP, WPE, SJ, K2, true>), dim3((unsigned)g.sk_wgs),
                               dim3(C::NT), 0, stream, g);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    } else {
        wgs = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN) * g.ksplit;
    }
    if (SJ > 0 && ((g.K / 64) + g.ksplit - 1) / g.ksplit > 4 * SJ) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemm_a16<TM, TN, WM, WN, NS, AF, EP, WPE, SJ, K2>), dim3((unsigned)wgs), dim3(C::NT), 0, stream, g);
    return hipGetLastError();
}

// The small-M tiles preload their scales when a workgroup's K range is at
// most 64 steps (4, 8 or 16 chunks per column, the fewest that cover it, so
// that little is read past the range), else they load them per step.
template <int TM, int TN, int WM, int WN, int NS, AFmt AF, Epi EP>
hipError_t launch_small(const GemmArgs& g, int grid_m, hipStream_t stream) {
    const int64_t per = ((g.K / 64) + g.ksplit - 1) / g.ksplit;
    if (per <= 16) return launch_cfg<TM, TN, WM, WN, NS, AF, EP, 1, 4, true>(g, grid_m, stream);
    if (per <= 32) return launch_cfg<TM, TN, WM, WN, NS, AF, EP, 1, 8, true>(g, grid_m, stream);
    if (per <= 64) return launch_cfg<TM, TN, WM, WN, NS, AF, EP, 1, 16, true>(g, grid_m, stream);
    return launch_cfg<TM, TN, WM, WN, NS, AF, EP>(g, grid_m, stream);
}

template <AFmt AF, Epi EP>
hipError_t launch_tile(const GemmArgs& g, A16Tile tile, int grid_m, hipStream_t stream) {
    switch (tile) {
        case A16Tile::k256x256_w128x64: return launch_cfg<4, 2, 2, 4, 3, AF, EP>(g, grid_m, stream);
        case A16Tile::k128x128_w64x64: return launch_cfg<2, 2, 2, 2, 2, AF, EP, 3>(g, grid_m, stream);
        case A16Tile::k128x128_w32x64: return launch_small<1, 2, 4, 2, 3, AF, EP>(g, grid_m, stream);
        case A16Tile::k64x256_w64x64: return launch_small<2, 2, 1, 4, 3, AF, EP>(g, grid_m, stream);
        case A16Tile::k32x256_w32x64: return launch_small<1, 2, 1, 4, 3, AF, EP>(g, grid_m, stream);
        case A16Tile::k192x128_w96x64: return launch_cfg<3, 2, 2, 2, 2, AF, EP, 2>(g, grid_m, stream);
    }
    return hipErrorInvalidValue;
}

// Split-K finish: y = bf16(scale * sum_s partial[s]) with the splits summed
// in order (s = 0 + p0 + p1 + ...).  KS is the split count, so that a thread
// issues all KS loads before its first add; V = 4 outputs per thread with
// 16-byte loads (M N % 4 == 0), else 1.
template <int KS, int V>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ partial, int64_t total,
                                                       const float* __restrict__ g0, const float* __restrict__ g1,
                                                       uint16_t* __restrict__ y, bool y8) {
    const float scale = *g0 * (g1 ? *g1 : 1.0f);
    const int64_t n = total / V;
    for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n; v += (int64_t)gridDim.x * 256) {
        if constexpr (V == 4) {
            f32x4 p[KS];
#pragma unroll
            for (int k = 0; k < KS; ++k) p[k] = *reinterpret_cast<const f32x4*>(partial + k * total + 4 * v);
            float s[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[e] = 0.0f;
#pragma unroll
                for (int k = 0; k < KS; ++k) s[e] += p[k][e];
            }
            uint32_t b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = f32_to_bf16_rne(s[e] * scale);
            if (y8) {
                *reinterpret_cast<uint2*>(y + 4 * v) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) y[4 * v + e] = (uint16_t)b[e];
            }
        } else {
            float p[KS];
#pragma unroll
            for (int k = 0; k < KS; ++k) p[k] = partial[k * total + v];
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < KS; ++k) s += p[k];
            y[v] = (uint16_t)f32_to_bf16_rne(s * scale);
        }
    }
}

// Stream-K finish.  Only tiles that a workgroup boundary cuts have parts to
// sum: the start x = floor(w S / wgs) of workgroup w (1 <= w < wgs) lies
// strictly inside tile t = x / ks.  Workgroup b of the launch takes boundary
// w = b / pieces + 1 and kSkRows rows (piece b % pieces) of that tile; when
// several boundaries cut one tile, the first of them does the work.  The
// tile's (tm, tn) follow the GEMM's band order; its K steps [t ks,
// (t + 1) ks) were shared by workgroups first(t) .. last(t), whose slots
// 0 .. last - first are summed in order.  V = 4 columns per thread (N % 4 ==
// 0, so a thread's columns lie in one row), else 1.
constexpr int kMaxSkSlots = 8;
constexpr int kSkRows = 32;
constexpr int kSkCols = 256;   // the tile width this finish is written for
template <int V>
__global__ __launch_bounds__(256) void k_streamk_reduce(const float* __restrict__ partial, int64_t M, int64_t N,
                                                        int ksteps, int wgs, int bm,
                                                        const float* __restrict__ g0, const float* __restrict__ g1,
                                                        uint16_t* __restrict__ y, bool y8) {
    constexpr int kTpr = kSkCols / V;              // threads per tile row
    constexpr int kPasses = kSkRows * kTpr / 256;  // rows per thread
    const int mtiles = (int)((M + bm - 1) / bm), ntiles = (int)((N + kSkCols - 1) / kSkCols);
    const int64_t S = (int64_t)mtiles * ntiles * ksteps;
    const int pieces = bm / kSkRows;
    const int bw = (int)(blockIdx.x / (unsigned)pieces) + 1, piece = (int)(blockIdx.x % (unsigned)pieces);
    const int64_t x = (int64_t)bw * S / wgs;
    if (x % ksteps == 0) return;                         // between two tiles
    const int t = (int)(x / ksteps);
    if ((int64_t)(bw - 1) * S / wgs > (int64_t)t * ksteps) return;   // an earlier boundary cuts this tile
    const int w0 = sk_first((int64_t)t * ksteps, wgs, S), w1 = sk_first((int64_t)(t + 1) * ksteps - 1, wgs, S);
    const int slots = w1 - w0 + 1;
    const int band = t / (kGroupM * ntiles), first_m = band * kGroupM;
    const int gsz = min(mtiles - first_m, kGroupM);
    const int r = t - band * kGroupM * ntiles;
    const int tm = first_m + r % gsz, tn = r / gsz;
    const float scale = *g0 * (g1 ? *g1 : 1.0f);
    const int64_t total = M * N;
    const int64_t col = (int64_t)tn * kSkCols + (int)(threadIdx.x % kTpr) * V;
    if (col >= N) return;
    const int64_t row0 = (int64_t)tm * bm + piece * kSkRows + threadIdx.x / kTpr;
    constexpr int kRowStep = 256 / kTpr;
    // all rows' loads of one slot are issued before they are added
    float sum[kPasses][V];
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps)
#pragma unroll
        for (int c = 0; c < V; ++c) sum[ps][c] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxSkSlots; ++k) {
        if (k >= slots) break;
        if constexpr (V == 4) {
            f32x4 v[kPasses];
#pragma unroll
            for (int ps = 0; ps < kPasses; ++ps) {
                const int64_t row = row0 + ps * kRowStep;
                v[ps] = row < M ? *reinterpret_cast<const f32x4*>(partial + k * total + row * N + col) : f32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int ps = 0; ps < kPasses; ++ps)
#pragma unroll
                for (int c = 0; c < 4; ++c) sum[ps][c] += v[ps][c];
        } else {
            float v[kPasses];
#pragma unroll
            for (int ps = 0; ps < kPasses; ++ps) {
                const int64_t row = row0 + ps * kRowStep;
                v[ps] = row < M ? partial[k * total + row * N + col] : 0.0f;
            }
#pragma unroll
            for (int ps = 0; ps < kPasses; ++ps) sum[ps][0] += v[ps];
        }
    }
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        const int64_t row = row0 + ps * kRowStep;
        if (row >= M) break;
        const int64_t e = row * N + col;
        if constexpr (V == 4) {
            uint32_t b[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) b[c] = f32_to_bf16_rne(sum[ps][c] * scale);
            if (y8) {
                *reinterpret_cast<uint2*>(y + e) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) y[e + c] = (uint16_t)b[c];
            }
        } else {
            y[e] = (uint16_t)f32_to_bf16_rne(sum[ps][0] * scale);
        }
    }
}

template <int KS>
hipError_t launch_reduce_ks(const float* partial, int64_t total, const float* g0, const float* g1, uint16_t* y,
                            hipStream_t stream) {
    const bool vec = (total % 4) == 0 && (reinterpret_cast<uintptr_t>(partial) & 15u) == 0;
    const int64_t n = vec ? total / 4 : total;
    int64_t grid = (n + 255) / 256;
    if (grid > 8192) grid = 8192;
    if (grid < 1) grid = 1;
    const bool y8 = (reinterpret_cast<uintptr_t>(y) & 7u) == 0;
    if (vec)
        hipLaunchKernelGGL((k_splitk_reduce<KS, 4>), dim3((unsigned)grid), dim3(256), 0, stream, partial, total, g0,
                           g1, y, y8);
    else
        hipLaunchKernelGGL((k_splitk_reduce<KS, 1>), dim3((unsigned)grid), dim3(256), 0, stream, partial, total, g0,
                           g1, y, y8);
    return hipGetLastError();
}

}  // namespace

int a16_tile_rows(A16Tile t) {
    switch (t) {
        case A16Tile::k256x256_w128x64: return 256;
        case A16Tile::k128x128_w64x64: return 128;
        case A16Tile::k128x128_w32x64: return 128;
        case A16Tile::k64x256_w64x64: return 64;
        case A16Tile::k32x256_w32x64: return 32;
        case A16Tile::k192x128_w96x64: return 192;
    }
    return 0;
}

int a16_tile_cols(A16Tile t) {
    switch (t) {
        case A16Tile::k256x256_w128x64: return 256;
        case A16Tile::k128x128_w64x64: return 128;
        case A16Tile::k128x128_w32x64: return 128;
        case A16Tile::k64x256_w64x64: return 256;
        case A16Tile::k32x256_w32x64: return 256;
        case A16Tile::k192x128_w96x64: return 128;
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
            if (tile != A16Tile::k192x128_w96x64) break;                                  \
            return launch_cfg<3, 2, 2, 2, 2, AF, Epi::kMoeGateUpLora, 2>(g, grid_m, stream); \
        case Epi::kMoeDownLora:                                                           \
            if (tile != A16Tile::k192x128_w96x64) break;                                  \
            return launch_cfg<3, 2, 2, 2, 2, AF, Epi::kMoeDownLora, 2>(g, grid_m, stream);   \
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
    const int64_t total = M * N;
    switch (ksplit) {
        case 2: return launch_reduce_ks<2>(partial, total, g0, g1, y, stream);
        case 3: return launch_reduce_ks<3>(partial, total, g0, g1, y, stream);
        case 4: return launch_reduce_ks<4>(partial, total, g0, g1, y, stream);
        case 5: return launch_reduce_ks<5>(partial, total, g0, g1, y, stream);
        case 6: return launch_reduce_ks<6>(partial, total, g0, g1, y, stream);
        case 7: return launch_reduce_ks<7>(partial, total, g0, g1, y, stream);
        case 8: return launch_reduce_ks<8>(partial, total, g0, g1, y, stream);
        case 9: return launch_reduce_ks<9>(partial, total, g0, g1, y, stream);
        case 10: return launch_reduce_ks<10>(partial, total, g0, g1, y, stream);
        case 11: return launch_reduce_ks<11>(partial, total, g0, g1, y, stream);
        case 12: return launch_reduce_ks<12>(partial, total, g0, g1, y, stream);
        case 13: return launch_reduce_ks<13>(partial, total, g0, g1, y, stream);
        case 14: return launch_reduce_ks<14>(partial, total, g0, g1, y, stream);
        case 15: return launch_reduce_ks<15>(partial, total, g0, g1, y, stream);
        case 16: return launch_reduce_ks<16>(partial, total, g0, g1, y, stream);
        default: return hipErrorInvalidValue;   // the split-K plans use 2 .. 16 splits
    }
}

}  // namespace nvfp4

namespace nvfp4 {

int streamk_slots(int64_t M, int64_t N, int64_t K, A16Tile tile, int wgs) {
    const int64_t bm = a16_tile_rows(tile), bn = a16_tile_cols(tile), ks = K / 64;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn), S = tiles * ks;
    if (wgs <= 0 || ks <= 0 || wgs > S) return 0;
    int most = 0;
    for (int64_t t = 0; t < tiles; ++t)
        most = std::max(most, sk_first((t + 1) * ks - 1, wgs, S) - sk_first(t * ks, wgs, S) + 1);
    return most;
}

hipError_t launch_streamk_reduce(const float* partial, int64_t M, int64_t N, int64_t K, A16Tile tile, int wgs,
                                 const float* g0, const float* g1, uint16_t* y, hipStream_t stream) {
    const int slots = streamk_slots(M, N, K, tile, wgs);
    if (slots < 1 || slots > kMaxSkSlots) return hipErrorInvalidValue;
    if (slots == 1) return hipSuccess;   // every tile was finished by the GEMM
    const int bm = a16_tile_rows(tile), bn = a16_tile_cols(tile);
    if (bm % kSkRows != 0 || bn != kSkCols || wgs < 2) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)(wgs - 1) * (bm / kSkRows);
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    const bool vec = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(partial) & 15u) == 0;
    const bool y8 = (reinterpret_cast<uintptr_t>(y) & 7u) == 0;
    if (vec)
        hipLaunchKernelGGL((k_streamk_reduce<4>), dim3((unsigned)grid), dim3(256), 0, stream, partial, M, N,
                           (int)(K / 64), wgs, bm, g0, g1, y, y8);
    else
        hipLaunchKernelGGL((k_streamk_reduce<1>), dim3((unsigned)grid), dim3(256), 0, stream, partial, M, N,
                           (int)(K / 64), wgs, bm, g0, g1, y, y8);
    return hipGetLastError();
}

}  // namespace nvfp4
