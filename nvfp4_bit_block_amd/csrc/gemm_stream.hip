// gemm_stream.hip -- small-batch NVFP4 GEMM that streams the weights:
// Y [M, N] = A [M, K] * W^T with W NVFP4 [N, K] and M <= 128.
//
// The weight-streaming regime of the W4A4 batch sweep and of W4A16 at
// small batch (model card "vroomfondel/glm-5.2-reap-504B-v2-W4A4", "Kernel
// choice"; Fprop with the contraction axis innermost, "Getting GLM-5.2 NVFP4
// Post-Training off the ground", "TN, NT, and what actually binds").  At
// these M the product is bound by the weight bytes, so the kernel is built
// like a GEMV that multiplies on the matrix cores:
//
//   * a workgroup (8 waves) owns BN = 16 NB weight rows and a range of K
//     (the whole K, or 1/S of it under a K split); the launcher sizes the
//     grid so that every workgroup is resident at once, and the weight
//     stream never waits for a second round of workgroups;
//   * the weights move from HBM straight into LDS (buffer_load ... lds, each
//     instruction 1 KB of two contiguous 512-byte row pieces, or 256 bytes of
//     scales), in chunks of 1024 K (512 K when up to 128 activation rows
//     share the stage) through an NS-stage ring, NS - 1 chunks in flight;
//     workgroups start at different chunks of their K range so that the
//     chip's concurrent reads spread over the rows;
//   * the activation slice a wave needs for the whole K range is either
//     loaded into registers once, in the prologue (so the ring's vmcnt waits
//     never wait on it): as 16-bit values (bf16 for W4A16, or the f16
//     products q * s of an already quantized activation), as packed NVFP4
//     codes and scale bytes decoded to exact f16 q * s at use, or as bf16
//     values that the wave quantizes in registers under the static input
//     scale with the quantizer's block rule (then kept as packed codes); or,
//     where it does not fit the registers (packed above 16 rows, bf16 on long
//     rows), streamed through the same ring beside the weights;
//   * K is split across the 8 waves (wave w takes K [128 w, 128 w + 128) of
//     every chunk, so each activation element is loaded once per
//     workgroup); a wave decodes its weight fragments from LDS to exact q * s
//     and runs v_mfma_f32_16x16x32_{f16,bf16} with the weights as the A
//     operand (16 weight rows) and the activation as B (16 batch rows);
//   * the eight wave partials meet in LDS and are summed in wave order; the
//     workgroup writes bf16 Y (scaled by both global scales) or, under a K
//     split, an fp32 partial that the split-K reduction sums in split order.
//
// K order: lane l of a 16x16x32 MFMA supplies row l % 16 of its operand at
// K group l / 16 (8 values).  The same K permutation is applied to both
// operands: in a wave's 128-K unit, lane group g takes the 32 consecutive K
// [32 g, 32 g + 32) (two NVFP4 blocks, 16 code bytes) and MFMA kk of the
// unit uses [32 g + 8 kk, +8).  A lane thus reads one 16-byte code chunk and
// two scale bytes per weight row block, and holds whole blocks of its own
// activation row.
//
// LDS layout of a stage: codes [BN rows][32 slots of 16 B], row r keeping
// its chunk u in slot u ^ (r % 8); scales [BN rows][16 dwords], row r
// keeping dword d in slot d ^ (r % 16).  Both keep the fragment reads of 16
// consecutive rows on distinct banks.
#include "nvfp4_device.hpp"
#include "nvfp4_dma.hpp"
#include "nvfp4_encode.hpp"
#include "nvfp4_internal.hpp"

#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kChunkK = 1024;          // K per ring stage of the register-activation forms

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word4(const uint4& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Eight weight codes -> eight MFMA operand values q * s (exact).
__device__ __forceinline__ f16x8 decode8(uint32_t w, _Float16 s, f16x8*) { return fp4x8_scaled_f16(w, s); }
__device__ __forceinline__ bf16x8 decode8(uint32_t w, float s, bf16x8*) {
    return __builtin_bit_cast(bf16x8, fp4x8_scaled_bf16_bits(w, s));
}
// Two E4M3 scale bytes (bits 0-7, 8-15) -> the pair in the decode's
// precision, through the exact FP8 -> fp32 conversion (every E4M3 value is
// an f16 value, so the narrowing is exact too).
__device__ __forceinline__ f16x2 scale_pair(uint32_t w, f16x8*) {
    const f32x2 f = e4m3x2_to_f32(w);
    return f16x2{(_Float16)f.x, (_Float16)f.y};
}
__device__ __forceinline__ f32x2 scale_pair(uint32_t w, bf16x8*) { return e4m3x2_to_f32(w); }

// Wait until at most n vector memory operations of this wave are in flight
// (n a multiple of the per-stage load count, at most NS - 2 stages).
template <int L>
__device__ __forceinline__ void wait_stages(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(L)); break;
        case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * L)); break;
        default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * L)); break;
    }
}

// NB: 16-row weight blocks per workgroup (2 or 4); MB: 16-row batch blocks
// (M <= 16 MB); NS: ring stages (2..5); NCH: the most 1024-K chunks a
// workgroup's K range may hold (sizes the activation registers); CK: K per
// ring stage (1024, or 512 so that up to 128 activation rows fit a stage;
// kPackedLds only).  The waves split a stage's K into WK = CK / 128 units of
// 128 and, when WK < 8, the batch blocks into 8 / WK groups.
template <int NB, int MB, SAct AM, int NS, int NCH, int CK = kChunkK>
__global__ __launch_bounds__(kThreads) void k_gemm_stream(StreamArgs g) {
    using Op = typename std::conditional<AM == SAct::kBf16 || AM == SAct::kBf16Lds, bf16x8, f16x8>::type;
    constexpr bool kPk = AM == SAct::kPacked || AM == SAct::kQuant;   // activation kept packed in registers
    constexpr bool kLdsP = AM == SAct::kPackedLds;                    // packed activation streamed through LDS
    constexpr bool kLdsB = AM == SAct::kBf16Lds;                      // bf16 activation streamed through LDS
    constexpr bool kLds = kLdsP || kLdsB;
    static_assert(CK == kChunkK || (kLds && CK == 512), "512-K stages stream the activation");
    constexpr int WK = CK / 128, WM = kWaves / WK, MBW = MB / WM;
    constexpr int RC = CK / 2, RSB = CK / 16;                 // code and scale bytes of a row per stage
    constexpr int NSLOT = RC / 16, NDW = RSB / 4;             // its 16-byte code slots and scale dwords
    constexpr int BN = 16 * NB, MP = kLds ? 16 * MB : 0;
    constexpr int RA = 2 * CK, LPR = RA / 1024;               // bf16 activation: bytes of a row per stage, loads per row
    constexpr int CODE_BYTES = BN * RC, WBYTES = BN * (RC + RSB);
    constexpr int ACODE = WBYTES, ASCALE = WBYTES + MP * RC;          // activation rows of a stage (kLds)
    // a load instruction of a wave covers 1 KB of codes (1024 / RC rows) or
    // 256 bytes of scales (256 / RSB rows); every wave issues the same number
    // of each kind, and one numbered past the last slab loads zeros into a
    // 1 KB pad at the end of the stage
    constexpr int NLC = BN * RC / 1024, NLS = BN * RSB / 256;
    constexpr int NLCA = kLdsB ? MP * LPR : MP * RC / 1024, NLSA = kLdsB ? 0 : MP * RSB / 256;
    constexpr int LC = (NLC + kWaves - 1) / kWaves, LS = (NLS + kWaves - 1) / kWaves;
    constexpr int LCA = (NLCA + kWaves - 1) / kWaves, LSA = (NLSA + kWaves - 1) / kWaves;
    constexpr bool kPad = LC * kWaves != NLC || LS * kWaves != NLS || LCA * kWaves != NLCA || LSA * kWaves != NLSA;
    constexpr int PAD = WBYTES + MP * (kLdsB ? RA : RC + RSB);
    constexpr int STAGE = PAD + (kPad ? 1024 : 0);
    constexpr int L = LC + LS + LCA + LSA;                    // DMA loads per wave per stage
    constexpr int ROWS = 16 * MB, RSTR = BN + 4;             // reduction buffer [K unit][row][RSTR] fp32
    constexpr int RED_BYTES = WK * ROWS * RSTR * 4;
    constexpr int LDS = NS * STAGE > RED_BYTES ? NS * STAGE : RED_BYTES;
    static_assert(NB == 2 || NB == 4, "weight row blocks");
    static_assert(!kLdsP || MB >= 2, "activation row blocks");
    static_assert(MB % WM == 0, "batch blocks per wave group");
    static_assert(NS >= 2 && NS <= 5 && LDS <= 160 * 1024, "LDS");
    static_assert(L * (NS - 2) <= 63, "vmcnt");
    __shared__ __align__(1024) uint8_t smem[LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = w % WK, wm = w / WK;                       // K unit and batch group of the wave
    const int i16 = lane & 15, grp = lane >> 4;

    const int64_t N = g.N, K = g.K, M = g.M;
    const int ntn = (int)((N + BN - 1) / BN);
    const int tn = (int)blockIdx.x % ntn, kz = (int)blockIdx.x / ntn;
    const int64_t n0 = (int64_t)tn * BN;
    const int64_t k0 = (int64_t)kz * g.krange;
    const int64_t k1 = min(K, k0 + g.krange);
    const int nchunks = (int)((k1 - k0 + CK - 1) / CK);   // 1 .. NCH (launcher; any count for kLds)
    const uint32_t KB = (uint32_t)(K / 2), KS = (uint32_t)(K / 16);
    const u32x4 rb_c = make_rsrc(g.b_codes, (uint64_t)N * KB);
    const u32x4 rb_s = make_rsrc(g.b_scales, (uint64_t)N * KS);
    const u32x4 ra_c = make_rsrc(kLds ? g.a : nullptr, kLdsB ? (uint64_t)M * K * 2 : kLds ? (uint64_t)M * KB : 0);
    const u32x4 ra_s = make_rsrc(kLds ? g.a_scales : nullptr, kLds ? (uint64_t)M * KS : 0);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(smem));

    // ---- 1. the first NS - 1 chunks of weights into the ring
    // Code load q = w LC + u covers rows (1024 / RC) q + lane / NSLOT, slot
    // lane % NSLOT <- the row's 16-byte chunk (lane % NSLOT) ^ (row % 8);
    // scale load q covers rows (256 / RSB) q + lane / NDW, dword slot
    // lane % NDW <- dword (lane % NDW) ^ (row % NDW).  The per-lane offsets of
    // the range's first chunk are computed once (an offset past every buffer
    // for pieces past N or M, which read zeros); a chunk adds its K offset.
    // Pieces past the K range are loaded but never multiplied: k1 is a
    // multiple of 128 and a wave skips any 128-K unit at or past it; past the
    // end of the last row they read zeros.
    // Workgroups start at different chunks of their range (chunk c of the
    // loop is chunk (c + rot) mod nchunks), so that the chip's concurrent
    // reads spread over the rows instead of all meeting at one K offset.
    const int rot = (int)(blockIdx.x % (unsigned)nchunks);
    auto rchunk = [&](int c) { return c + rot < nchunks ? c + rot : c + rot - nchunks; };   // c < nchunks
    constexpr int RPC = 1024 / RC, RPS = 256 / RSB;
    constexpr int NOCA = kLds ? LCA : 1, NOSA = kLdsP ? LSA : 1;
    uint32_t oc[LC], os[LS], oca[NOCA], osa[NOSA];
    auto code_off = [&](int q, int nq, int64_t row0, int64_t rows) -> uint32_t {
        const int r = RPC * q + lane / NSLOT;
        const int unit = (lane % NSLOT) ^ (r & 7);
        const int64_t row = row0 + r;
        return q < nq && row < rows ? (uint32_t)row * KB + (uint32_t)((k0 + 32 * unit) / 2) : kOob;
    };
    auto scale_off = [&](int q, int nq, int64_t row0, int64_t rows) -> uint32_t {
        const int r = RPS * q + lane / NDW;
        const int d = (lane % NDW) ^ (r & (NDW - 1));
        const int64_t row = row0 + r;
        return q < nq && row < rows ? (uint32_t)row * KS + (uint32_t)((k0 + 64 * d) / 16) : kOob;
    };
#pragma unroll
    for (int u = 0; u < LC; ++u) oc[u] = code_off(w * LC + u, NLC, n0, N);
#pragma unroll
    for (int u = 0; u < LS; ++u) os[u] = scale_off(w * LS + u, NLS, n0, N);
    if constexpr (kLdsP) {
#pragma unroll
        for (int u = 0; u < LCA; ++u) oca[u] = code_off(w * LCA + u, NLCA, 0, M);
#pragma unroll
        for (int u = 0; u < LSA; ++u) osa[u] = scale_off(w * LSA + u, NLSA, 0, M);
    }
    if constexpr (kLdsB) {
        // bf16 activation rows, RA bytes each: load q fills 1 KB of row
        // q / LPR, slot p (16 bytes, 8 values) <- the row's slot p ^ (row % 16),
        // which spreads the fragment reads of 16 consecutive rows over the
        // banks (the swizzle stays inside a 128-K unit of 16 slots)
#pragma unroll
        for (int u = 0; u < LCA; ++u) {
            const int q = w * LCA + u, r = q / LPR;
            const int slot = 64 * (q % LPR) + lane;
            oca[u] = q < NLCA && r < M ? (uint32_t)((r * K + k0 + 8 * (slot ^ (r & 15))) * 2) : kOob;
        }
    }
    auto issue = [&](int c, int st) {
        const uint32_t base = lds0 + (uint32_t)(st * STAGE), pad = base + (uint32_t)PAD;
        const uint32_t dk = (uint32_t)(rchunk(c) * CK);   // K offset of the chunk in the range
#pragma unroll
        for (int u = 0; u < LC; ++u) {
            const int q = w * LC + u;
            lds_load16(rb_c, oc[u] + dk / 2, 0u, q < NLC ? base + (uint32_t)(q * 1024) : pad);
        }
#pragma unroll
        for (int u = 0; u < LS; ++u) {
            const int q = w * LS + u;
            lds_load4(rb_s, os[u] + dk / 16, 0u, q < NLS ? base + (uint32_t)(CODE_BYTES + q * 256) : pad);
        }
        if constexpr (kLdsP) {
            // the chunk's activation rows, laid out like the weight rows
#pragma unroll
            for (int u = 0; u < LCA; ++u) {
                const int q = w * LCA + u;
                lds_load16(ra_c, oca[u] + dk / 2, 0u, q < NLCA ? base + (uint32_t)(ACODE + q * 1024) : pad);
            }
#pragma unroll
            for (int u = 0; u < LSA; ++u) {
                const int q = w * LSA + u;
                lds_load4(ra_s, osa[u] + dk / 16, 0u, q < NLSA ? base + (uint32_t)(ASCALE + q * 256) : pad);
            }
        }
        if constexpr (kLdsB) {
#pragma unroll
            for (int u = 0; u < LCA; ++u) {
                const int q = w * LCA + u;
                lds_load16(ra_c, oca[u] + 2 * dk, 0u, q < NLCA ? base + (uint32_t)(ACODE + q * 1024) : pad);
            }
        }
    };
    if constexpr (AM != SAct::kQuant) {
#pragma unroll
        for (int s = 0; s + 1 < NS; ++s)
            if (s < nchunks) issue(s, s);
    }

    // ---- 2. activation loads: this wave's 128-K unit of every chunk, rows
    // 16 mb + i16, as unconditional buffer loads (zeros past M or past the K
    // range), then one wait for everything issued so far.  (The compiler
    // tracks these loads but not the asm weight loads, so the first use of
    // the activation has to follow a full wait; from here on the K loop
    // issues weight loads only and waits for them itself.)
    constexpr int XN = (kPk || kLds) ? 1 : NCH, XM = (kPk || kLds) ? 1 : MB;
    constexpr int QN = AM == SAct::kQuant ? NCH : 1, QM = AM == SAct::kQuant ? MB : 1;
    constexpr int PN = kPk ? NCH : 1, PM = kPk ? MB : 1;
    uint4 xa[XN][XM][4];      // 16-bit activation values (kBf16, kF16)
    uint4 xq[QN][QM][4];      // bf16 staging of the in-register quantization (kQuant)
    uint4 xc[PN][PM];         // packed codes (kPacked, kQuant)
    uint32_t xs[PN][PM];      // their two scale bytes
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.a), (short)0, (int)(AM == SAct::kPacked ? M * K / 2 : M * K * 2), (int)kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.a_scales), (short)0, (int)(AM == SAct::kPacked ? M * K / 16 : 0), (int)kRsrcWord3);
#pragma unroll
    for (int c = 0; c < (kLds ? 0 : NCH); ++c) {
        const int64_t ku = k0 + (int64_t)rchunk(c) * kChunkK + 128 * w;   // the wave's unit (uniform)
        const bool kin = c < nchunks && ku < k1;
        const int64_t ka = ku + 32 * grp;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int64_t m = 16 * mb + i16;
            const bool in = kin && m < M;
            if constexpr (AM == SAct::kPacked) {
                const uint32_t oc = in ? (uint32_t)(m * (K / 2) + ka / 2) : kOob;
                const uint32_t os = in ? (uint32_t)(m * (K / 16) + ka / 16) : kOob;
                xc[c][mb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, oc, 0, 0));
                xs[c][mb] = __builtin_amdgcn_raw_buffer_load_b16(ras, os, 0, 0);
            } else {
                const uint32_t o = in ? (uint32_t)((m * K + ka) * 2) : kOob;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint4 v = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, in ? o + 16u * p : kOob, 0, 0));
                    if constexpr (AM == SAct::kQuant) xq[c][mb][p] = v;
                    else xa[c][mb][p] = v;
                }
            }
        }
    }
    if constexpr (kLds) wait_stages<L>(min(NS - 2, nchunks - 1));   // chunk 0 only: all loads are DMA
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // ---- 3. in-register quantization (kQuant): the weights are issued only
    // now (the activation has landed), so the encode runs while they
    // stream; each lane encodes its two 16-element blocks per unit under the
    // static scale
    if constexpr (AM == SAct::kQuant) {
#pragma unroll
        for (int s = 0; s + 1 < NS; ++s)
            if (s < nchunks) issue(s, s);
        const float sg = *g.a_global, t = 6.0f * sg;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                uint32_t s2 = 0;
                uint2 c0 = make_uint2(0, 0), c1 = make_uint2(0, 0);
                const uint4* v = xq[c][mb];
                const uint32_t b0[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
                const uint32_t b1[8] = {v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
                s2 = encode_block(b0, sg, t, c0);
                s2 |= encode_block(b1, sg, t, c1) << 8;
                xc[c][mb] = make_uint4(c0.x, c0.y, c1.x, c1.y);
                xs[c][mb] = s2;
            }
        wait_stages<L>(min(NS - 2, nchunks - 1));
    }
    __syncthreads();

    // ---- 4. the K loop
    f32x4 acc[NB][MBW];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) acc[nb][mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t fcode = (uint32_t)(i16 * RC + 16 * ((4 * wk + grp) ^ (i16 & 7)));
    const uint32_t fscale =
        (uint32_t)(CODE_BYTES + i16 * RSB + 4 * ((2 * wk + (grp >> 1)) ^ (i16 & (NDW - 1))) + 2 * (grp & 1));

    // (the wave's batch blocks are wm MBW .. wm MBW + MBW - 1; with the
    // activation in registers WM = 1 and they are all MB)
    // the wave's fragments of one chunk, read from its ring stage
    using Sc = typename std::conditional<std::is_same<Op, f16x8>::value, f16x2, f32x2>::type;
    constexpr int FP = kLdsP ? MBW : 1, FB = kLdsB ? MBW : 1;
    // (scale bytes stay raw here: converting them would make the wave wait
    // for its LDS reads before it issues the next chunk's loads)
    struct Frag {
        uint4 cw[NB];       // weight codes
        uint32_t sw[NB];    // their two block scales
        uint4 xl[FP];       // packed activation codes (kPackedLds)
        uint32_t xsc[FP];   // and scales
        uint4 xb[FB][4];    // bf16 activation operands (kBf16Lds)
    };
    auto fetch = [&](int st) {
        const uint8_t* sb = smem + st * STAGE;
        Frag f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            f.cw[nb] = *reinterpret_cast<const uint4*>(sb + fcode + nb * 16 * RC);
            f.sw[nb] = *reinterpret_cast<const uint16_t*>(sb + fscale + nb * 16 * RSB);
        }
        if constexpr (kLdsP) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                const int b = wm * MBW + mb;
                f.xl[mb] = *reinterpret_cast<const uint4*>(sb + ACODE + fcode + b * 16 * RC);
                f.xsc[mb] = *reinterpret_cast<const uint16_t*>(sb + ASCALE + (fscale - CODE_BYTES) + b * 16 * RSB);
            }
        }
        if constexpr (kLdsB) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    f.xb[mb][kk] = *reinterpret_cast<const uint4*>(
                        sb + ACODE + (16 * (wm * MBW + mb) + i16) * RA + 16 * ((16 * wk + 4 * grp + kk) ^ i16));
        }
        return f;
    };
    auto multiply = [&](int c, const Frag& f) {
        f16x2 xsc[(kPk || kLdsP) ? MBW : 1];
        Sc sw[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sw[nb] = scale_pair(f.sw[nb], (Op*)nullptr);
        if constexpr (kPk || kLdsP) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                if constexpr (kPk) xsc[mb] = scale_pair(xs[c][mb], (f16x8*)nullptr);
                else xsc[mb] = scale_pair(f.xsc[mb], (f16x8*)nullptr);
            }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            Op bx[MBW];
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                if constexpr (kPk) bx[mb] = fp4x8_scaled_f16(word4(xc[c][mb], kk), kk < 2 ? xsc[mb].x : xsc[mb].y);
                else if constexpr (kLdsP)
                    bx[mb] = fp4x8_scaled_f16(word4(f.xl[mb], kk), kk < 2 ? xsc[mb].x : xsc[mb].y);
                else if constexpr (kLdsB) bx[mb] = __builtin_bit_cast(Op, f.xb[mb][kk]);
                else bx[mb] = __builtin_bit_cast(Op, xa[c][mb][kk]);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const Op av = decode8(word4(f.cw[nb], kk), kk < 2 ? sw[nb].x : sw[nb].y, (Op*)nullptr);
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) acc[nb][mb] = mfma16(av, bx[mb], acc[nb][mb]);
            }
        }
    };

    // read chunk c's fragments, refill the stage multiplied in iteration
    // c - 1 (all waves passed the barrier after it) while they arrive,
    // multiply chunk c, wait for chunk c + 1
    auto iteration = [&](int c, int cr) {
        const bool mine = k0 + (int64_t)rchunk(c) * CK + 128 * wk < k1;
        Frag f;
        if (mine) f = fetch(c % NS);
        if (c + NS - 1 < nchunks) issue(c + NS - 1, (c + NS - 1) % NS);
        if (mine) multiply(cr, f);
        if (c + 1 < nchunks) {
            wait_stages<L>(min(NS - 2, nchunks - 2 - c));
            __syncthreads();
        }
    };
    if constexpr (kLds) {
        // no activation registers to index: a plain loop over any chunk count
        for (int c = 0; c < nchunks; ++c) iteration(c, 0);
    } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            if (c < nchunks) iteration(c, c);
    }

    // ---- 5. wave partials -> LDS (the ring is free once every wave is here),
    // one plane per K unit
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
            *reinterpret_cast<f32x4*>(red + (wk * ROWS + 16 * (wm * MBW + mb) + i16) * RSTR + 16 * nb + 4 * grp) =
                acc[nb][mb];
    __syncthreads();

    // ---- 6. sum in K-unit order; thread e takes batch row e / (BN/4) and four
    // consecutive weight rows
    constexpr int NG = BN / 4;
    const float scale = (g.a_global ? *g.a_global : 1.0f) * *g.b_global;
    for (int e = tid; e < ROWS * NG; e += kThreads) {
        const int mr = e / NG, ng = e - mr * NG;
        f32x4 s = *reinterpret_cast<const f32x4*>(red + mr * RSTR + 4 * ng);
#pragma unroll
        for (int v = 1; v < WK; ++v) s += *reinterpret_cast<const f32x4*>(red + (v * ROWS + mr) * RSTR + 4 * ng);
        const int64_t m = mr, n = n0 + 4 * ng;
        if (m >= M || n >= N) continue;
        if (g.ksplit > 1) {
            float* o = reinterpret_cast<float*>(g.out) + ((int64_t)kz * M + m) * N + n;
            if (n + 4 <= N && (N & 3) == 0) {
                *reinterpret_cast<f32x4*>(o) = s;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) o[r] = s[r];
            }
        } else {
            uint16_t* o = reinterpret_cast<uint16_t*>(g.out) + m * N + n;
            const uint32_t b0 = f32_to_bf16_rne(s[0] * scale), b1 = f32_to_bf16_rne(s[1] * scale);
            const uint32_t b2 = f32_to_bf16_rne(s[2] * scale), b3 = f32_to_bf16_rne(s[3] * scale);
            if (n + 4 <= N && (N & 3) == 0) {
                *reinterpret_cast<uint2*>(o) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
            } else {
                const uint32_t b[4] = {b0, b1, b2, b3};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) o[r] = (uint16_t)b[r];
            }
        }
    }
}

constexpr int kActBudget = 128;   // activation VGPRs per wave
constexpr int act_regs(SAct am, int mb) {
    return am == SAct::kPackedLds || am == SAct::kBf16Lds ? 0 : (am == SAct::kPacked ? 5 : 16) * mb;
}

// Bytes of one ring stage of the LDS-streamed forms (weight and activation
// rows, and the 1 KB pad when the loads do not divide evenly among the waves).
template <int NB, int MB, int CK, bool BF16>
constexpr int lds_stage_bytes() {
    constexpr int RC = CK / 2, RSB = CK / 16, BN = 16 * NB, MP = 16 * MB;
    constexpr int nla = BF16 ? MP * CK * 2 / 1024 : MP * RC / 1024, nlsa = BF16 ? 0 : MP * RSB / 256;
    constexpr bool pad = (BN * RC / 1024) % kWaves || (BN * RSB / 256) % kWaves || nla % kWaves || nlsa % kWaves;
    return BN * (RC + RSB) + (BF16 ? MP * CK * 2 : MP * (RC + RSB)) + (pad ? 1024 : 0);
}

template <int NB, int MB, SAct AM, int NCH>
hipError_t launch_one(const StreamArgs& g, hipStream_t stream) {
    constexpr bool kLds = AM == SAct::kPackedLds || AM == SAct::kBf16Lds;
    // LDS-streamed forms: 512-K stages above 64 packed or 16 bf16 batch rows,
    // and as many stages (up to four) as LDS holds
    constexpr int CK = (AM == SAct::kPackedLds && MB > 4) || (AM == SAct::kBf16Lds && MB > 1) ? 512 : kChunkK;
    constexpr int kLdsStage = lds_stage_bytes<NB, MB, CK, AM == SAct::kBf16Lds>();
    if constexpr (NCH * act_regs(AM, MB) > kActBudget || (AM == SAct::kPackedLds && MB < 2) ||
                  (kLds && 2 * kLdsStage > 160 * 1024)) {
        return hipErrorInvalidValue;
    } else {
        constexpr int NS = kLds ? (4 * kLdsStage <= 160 * 1024 ? 4 : 3 * kLdsStage <= 160 * 1024 ? 3 : 2)
                                : NCH == 1 ? 2 : NCH == 2 ? 3 : 4;
        const int64_t ntn = (g.N + 16 * NB - 1) / (16 * NB);
        hipLaunchKernelGGL((k_gemm_stream<NB, MB, AM, NS, NCH, CK>), dim3((unsigned)(ntn * g.ksplit)),
                           dim3(kThreads), 0, stream, g);
        return hipGetLastError();
    }
}

template <int NB, int MB, SAct AM>
hipError_t launch_nch(const StreamArgs& g, int nch, hipStream_t stream) {
    switch (nch) {
        case 1: return launch_one<NB, MB, AM, 1>(g, stream);
        case 2: return launch_one<NB, MB, AM, 2>(g, stream);
        case 4: return launch_one<NB, MB, AM, 4>(g, stream);
        case 8: return launch_one<NB, MB, AM, 8>(g, stream);
        case 16: return launch_one<NB, MB, AM, 16>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

template <SAct AM>
hipError_t launch_am(const StreamArgs& g, int nb, int mb, int nch, hipStream_t stream) {
    if (nb == 4) {
        switch (mb) {
            case 1: return launch_nch<4, 1, AM>(g, nch, stream);
            case 2: return launch_nch<4, 2, AM>(g, nch, stream);
            case 4: return launch_nch<4, 4, AM>(g, nch, stream);
        }
    } else if (nb == 2) {
        switch (mb) {
            case 1: return launch_nch<2, 1, AM>(g, nch, stream);
            case 2: return launch_nch<2, 2, AM>(g, nch, stream);
            case 4: return launch_nch<2, 4, AM>(g, nch, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Activation register budget per wave (kActBudget): 16 VGPRs per batch
// block and chunk for 16-bit values, 5 for packed codes (the in-register
// quantization stages 16 per block and chunk until it has encoded them).
int stream_max_chunks(SAct am, int mb) {
    if (am == SAct::kPackedLds || am == SAct::kBf16Lds) return 1 << 20;   // no activation registers: any chunk count
    int nch = 1;
    while (nch * 2 <= 16 && nch * 2 * act_regs(am, mb) <= kActBudget) nch *= 2;
    return nch;
}

hipError_t launch_gemm_stream(const StreamArgs& g, SAct am, int nb, int mb, hipStream_t stream) {
    if (g.K % 128 != 0 || g.krange % 128 != 0 || g.krange <= 0 || g.ksplit < 1) return hipErrorInvalidValue;
    if (g.M < 1 || g.M > 16 * mb) return hipErrorInvalidValue;
    const int64_t chunks = (g.krange + kChunkK - 1) / kChunkK;
    int nch = 1;
    while (nch < chunks) nch *= 2;
    if (nch > stream_max_chunks(am, mb)) return hipErrorInvalidValue;
    if (am == SAct::kPackedLds) {
        if (nb == 4) return mb == 2 ? launch_one<4, 2, SAct::kPackedLds, 1>(g, stream)
                          : mb == 4 ? launch_one<4, 4, SAct::kPackedLds, 1>(g, stream)
                          : mb == 8 ? launch_one<4, 8, SAct::kPackedLds, 1>(g, stream) : hipErrorInvalidValue;
        if (nb == 2) return mb == 2 ? launch_one<2, 2, SAct::kPackedLds, 1>(g, stream)
                          : mb == 4 ? launch_one<2, 4, SAct::kPackedLds, 1>(g, stream)
                          : mb == 8 ? launch_one<2, 8, SAct::kPackedLds, 1>(g, stream) : hipErrorInvalidValue;
        return hipErrorInvalidValue;
    }
    if (am == SAct::kBf16Lds) {
        if (nb == 4) return mb == 1 ? launch_one<4, 1, SAct::kBf16Lds, 1>(g, stream)
                          : mb == 2 ? launch_one<4, 2, SAct::kBf16Lds, 1>(g, stream)
                          : mb == 4 ? launch_one<4, 4, SAct::kBf16Lds, 1>(g, stream) : hipErrorInvalidValue;
        if (nb == 2) return mb == 1 ? launch_one<2, 1, SAct::kBf16Lds, 1>(g, stream)
                          : mb == 2 ? launch_one<2, 2, SAct::kBf16Lds, 1>(g, stream)
                          : mb == 4 ? launch_one<2, 4, SAct::kBf16Lds, 1>(g, stream) : hipErrorInvalidValue;
        return hipErrorInvalidValue;
    }
    switch (am) {
        case SAct::kBf16: return launch_am<SAct::kBf16>(g, nb, mb, nch, stream);
        case SAct::kF16: return launch_am<SAct::kF16>(g, nb, mb, nch, stream);
        case SAct::kPacked: return launch_am<SAct::kPacked>(g, nb, mb, nch, stream);
        case SAct::kQuant: return launch_am<SAct::kQuant>(g, nb, mb, nch, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace nvfp4
