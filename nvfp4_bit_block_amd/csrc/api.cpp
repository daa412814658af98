// api.cpp -- the C ABI declared in include/nvfp4.h: argument checks on the
// host, workspace layout, and the launch sequence of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>

#include "nvfp4.h"
#include "nvfp4_internal.hpp"

using namespace nvfp4;

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t status, const char* fmt, const char* detail = "") {
    std::snprintf(g_last_error, sizeof g_last_error, fmt, detail);
    return status;
}

int32_t hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return NVFP4_OK;
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(e));
    return NVFP4_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ----------------------------------------------------------- GEMM planning --

int64_t gemm_chunk_rows(int64_t M, int64_t K);

struct GemmPlan {
    bool gemv = false;   // M <= 8: decoded activation + GEMV
    A16Tile tile = A16Tile::k256x256_w128x64;
    int ksplit = 1;   // K splits, or with stream-K the partial slots
    int sk_wgs = 0;   // stream-K workgroups (0: none)
};

// Tile and split-K choice for the W4A4 GEMM (measured on MI355X: the
// 256x256 tile with eight 128x64 waves is the fastest per tile; smaller tiles
// win where 256x256 leaves most CUs idle; small M streams the weights once
// and splits K to spread that stream over the chip).
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool bf16_a = false) {
    GemmPlan p;
    // The VALU GEMV wins while its activation slice fits in registers (M <= 4,
    // the K = 2048 layout up to M = 8) or in LDS (short rows); beyond that the
    // MFMA tiles are faster.  On o_proj (K = 16384) the GEMV costs about 3 us
    // per row (19 us at M = 4, 31 us at M = 8) while the 32-row tile with its
    // scale preload costs about 26 us at any M up to 32, so the tile takes
    // M >= 7 there (M = 8: W4A4 35.6 -> 26.0 us, W4A16 31.5 -> 26.3 us).
    if (M <= 4 || (M <= 8 && K <= 4096) || (M <= 6 && K > 4096)) {
        p.gemv = true;
        return p;
    }
    const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
    // Short rows with enough tiles for every CU: the thin tiles need no K
    // split (measured on MI355X, q_b_proj 16384 x 2048: M = 128 on 32 x 256
    // tiles 19.1 us against 24.0 us for 128 x 128 tiles split in two plus the
    // split-K pass; M = 256 on the 128 x 128 tile with 32-row waves 26.6
    // against 28.2 us, f16 activation; with the bf16 activation of W4A16 that
    // tile loses, 34.2 against 31.5 us)
    const bool short_k = K <= 4096;
    // Long rows above M = 128: the 256 x 256 tile (its software-pipelined
    // 128-row waves) with K split until about one workgroup per CU beats the
    // 128 x 128 tiles (measured on MI355X, o_proj 6144 x 16384, f16 / bf16
    // activation: M = 256 72.4 / 87.5 -> 69.9 / 74.2 us at split 8; M = 512
    // 127.2 / 161.6 -> 116.6 / 123.8 at split 4; M = 1024 241.8 / 268.7 ->
    // 207.7 / 235.9 at split 2; M = 2048 445 -> 419 us unsplit).  On short
    // rows it needs 192 tiles of its own (q_b_proj M = 512: 128 x 128 tiles
    // 42.1 us against 55.9).
    const bool long_wide = !short_k && M > 128;
    if (short_k && M > 64 && M <= 128 && ((M + 31) / 32) * ((N + 255) / 256) >= 256) p.tile = A16Tile::k32x256_w32x64;
    else if (!bf16_a && short_k && M > 64 && M <= 256 && ((M + 127) / 128) * ((N + 127) / 128) >= 256)
        p.tile = A16Tile::k128x128_w32x64;
    else if (M <= 32) p.tile = A16Tile::k32x256_w32x64;
    // 32 < M <= 64: for short K the 128-row tile with 32-row waves (q_b_proj,
    // K = 2048: 22.6 us against 25.4 us with 64 x 256); for long K 64 x 256
    else if (M <= 64) p.tile = K <= 4096 ? A16Tile::k128x128_w32x64 : A16Tile::k64x256_w64x64;
    else if (long_wide || (M > 128 && big >= 192)) p.tile = A16Tile::k256x256_w128x64;
    else p.tile = A16Tile::k128x128_w64x64;
    const int64_t bm = a16_tile_rows(p.tile), bn = a16_tile_cols(p.tile);
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int64_t ksteps = K / 64;
    // split K until about one workgroup per CU.  Up to M = 64, and for the
    // 256 x 256 tile on long rows, the split stops at 256 workgroups and may
    // take any count: measured at M = 32 and 64 on o_proj (6144 x 16384), 192
    // workgroups (split 8) beat 384 (split 16) by 7-14 %, each further split
    // adding a partial-sum pass over M x N and a workgroup prologue for the
    // same weight stream; the 256 x 256 tile needs its one workgroup per CU
    // (M = 256: split 8 69.9 us against split 4 100.1 us; M = 2048 unsplit
    // 419 against split 2 445 us).
    const bool one_per_cu = long_wide && p.tile == A16Tile::k256x256_w128x64;
    if (one_per_cu || M <= 64) {
        // as many workgroups as fit one per CU, with any split count: 256 / tiles
        // (measured on MI355X, o_proj 6144 x 16384, f16 / bf16 activation: M = 256
        // split 10 (240 workgroups) 68.3 / 72.3 us against split 8 71.1 / 75.8;
        // M = 512 split 5 107.4 / 114.4 against split 4 118.8 / 125.2; M = 32 on
        // 32 x 256 tiles split 10 22.9 / 26.4 against split 8 23.4 / 27.9; M = 64
        // on 64 x 256 tiles 30.7 / 34.1 against 31.5 / 35.7)
        if (tiles < 256) p.ksplit = (int)std::min<int64_t>(16, 256 / tiles);
        while (p.ksplit > 1 && ksteps / p.ksplit < 8) --p.ksplit;
    } else {
        while (tiles * p.ksplit < 256 && p.ksplit < 16 && ksteps / (p.ksplit * 2) >= 8) p.ksplit *= 2;
    }
    // 256-511 tiles on long K leave some CUs one tile and others two (o_proj
    // at M = 4096: 384 tiles of 256 x 256, one per CU, so 1.5 rounds; 128 x
    // 128 grids of that size, three workgroups per CU); split 2 evens the
    // load (M = 4096: W4A4 814 -> 767 us, W4A16 861 -> 801; a 384-tile
    // 128 x 128 grid at M = 1024: 246.6 -> 234.2 us).  Short K, more tiles or
    // further splits measured slower: each split adds a partial-sum pass.
    if ((p.tile == A16Tile::k128x128_w64x64 || p.tile == A16Tile::k256x256_w128x64) && p.ksplit == 1 &&
        tiles >= 256 && tiles < 512 && ksteps >= 128)
        p.ksplit = 2;
    // Stream-K for the 256 x 256 tile on long rows: 256 workgroups share the
    // tiles' K steps evenly, a workgroup holding a whole tile writes it
    // finished, and the other tiles' parts are summed in order afterwards.
    // The chip does not run 256 busy CUs much faster than 192, and the
    // finish reads every part, so below 256 tiles it pays only where the
    // split leaves about 30 % of the CUs idle (measured on MI355X, o_proj
    // 6144 x 16384, f16 / bf16 activation: M = 1536, 144 workgroups
    // unsplit, 359.7 / 376.2 -> 306.6 / 319.0 us; M = 1024, 192 at split 2,
    // 227.5 / 227.5 -> 222.2 / 223.8; M = 2048, 192 unsplit, 382.0 / 417.4
    // -> 387.2 / 407.0; M = 768, 216 at split 3, 156.7 / 166.8 -> 161.6 /
    // 173.3).  With 256-511 tiles it replaces split 2 (same box, four runs
    // each: M = 4096 696.8 / 742.2 -> 681.6 / 727.5 us, M = 3072 604.0 /
    // 656.2 -> 582.8 / 618.3; on short rows, q_b_proj's 1024 tiles of 32
    // steps, it lost 4-6 % to the plain grid).  One launch (the rows fit one
    // buffer resource), at least 8 K steps per workgroup.
    const bool sk_idle = tiles * p.ksplit <= 176;
    const bool sk_rounds = tiles >= 256 && tiles < 512 && ksteps >= 128;
    if (one_per_cu && (sk_idle || sk_rounds) && gemm_chunk_rows(M, K) >= M && tiles * ksteps >= 256 * 8) {
        const int slots = streamk_slots(M, N, K, p.tile, 256);
        if (slots >= 1 && slots <= 8) {
            p.sk_wgs = 256;
            p.ksplit = slots;   // partial slots (one: every tile is written whole)
        }
    }
    return p;
}

// The weight-streaming MFMA kernel (gemm_stream.hip) for small batches.
// Measured on MI355X with NVFP4 weights rotated through HBM: where a weight
// row holds at most four 1024-K chunks (q_b_proj, 16384 x 2048) it beats
// both the GEMV (from M = 3) and the LDS-staged tiles up to M = 64 (W4A4 on
// a packed activation: M = 8 16.3 -> 7.9 us, M = 32 22.9 -> 10.0 us,
// M = 64 23.1 -> 13.7 us; W4A16 M = 8 15.1 -> 8.5 us, M = 64 22.1 ->
// 17.8 us); on long rows (o_proj, 6144 x 16384) it wins for the packed
// activation at M = 5..16 (M = 8 25.3 -> 21.2 us, M = 16 26.2 -> 22.6 us)
// and not for bf16 activations, whose registers limit a workgroup to half
// the row.
struct StreamPlan {
    bool use = false;
    SAct am = SAct::kPacked;
    int nb = 4, mb = 1, ksplit = 1;
    int64_t krange = 0;
};

// For a packed activation above M = 16 the activation is streamed through
// LDS with the weights (M = 65-128 on short rows only) (measured on MI355X: q_b_proj M = 32 / 64 10.0 ->
// 9.0 / 13.7 -> 11.7 us against the activation in registers; o_proj M = 32
// 27.9 -> 22.8 us and M = 64 36.7 -> 31.3 us against the tiles).
StreamPlan plan_stream(int64_t M, int64_t N, int64_t K, SAct am) {
    StreamPlan p;
    if (M < 1 || M > 128 || N < 1 || K % 128 != 0 || N * (K / 2) >= kMaxOperandBytes || M * K * 2 >= kMaxOperandBytes)
        return p;
    const bool short_k = K <= 4096;
    const bool lds = am == SAct::kPacked && M > 16;
    // bf16 activation on long rows, 5-16 batch rows: streamed through LDS
    // (measured on MI355X, o_proj 6144 x 16384: 22.9-23.3 us against 23.4
    // (GEMV, M = 5), 26.8 (tile, M = 8) and 27.1 us (tile, M = 16); with
    // 32 or 64 rows its 512-K stages lose to the tiles, 37 / 49 against 28 /
    // 37 us)
    const bool lds_b = am == SAct::kBf16 && !short_k && M >= 5 && M <= 16;
    if (short_k ? M < 3
                : (am == SAct::kQuant || M < 5 || (am == SAct::kBf16 && !lds_b) || (am != SAct::kBf16 && M > 16 && !lds)))
        return p;
    p.am = lds ? SAct::kPackedLds : lds_b ? SAct::kBf16Lds : am;
    p.mb = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
    auto krange_of = [&](int s) { return ((K / 128 + s - 1) / s) * 128; };
    if (lds_b) {
        // the fewest K splits first (each adds a partial-sum pass), then the
        // wider weight tile: o_proj takes 32-row tiles unsplit (23.2 us at
        // M = 8, against 24.6 us for 64-row tiles split in two)
        for (int s = 1; s <= 8 && K / 128 >= s; s *= 2)
            for (int nb = 4; nb >= 2; nb -= 2) {
                if (((N + 16 * nb - 1) / (16 * nb)) * s < 192) continue;
                p.use = true;
                p.nb = nb;
                p.ksplit = s;
                p.krange = krange_of(s);
                return p;
            }
        return p;
    }
    if (M > 64) {
        // 65-128 rows (512-K stages), 64-row weight tiles, the fewest K splits
        // (one or two) that give 192 workgroups (measured on MI355X: q_b_proj
        // M = 96 / 128 unsplit 30.6 / 23.6 -> 16.3 / 16.9 us; o_proj 6144 x
        // 16384, pre-packed activation, split 2: 50.4 / 52.0 -> 46.8 / 47.0 us,
        // where split 1 took 77 us and splits 4 and 8 49-52 us)
        if (!lds) return p;
        for (int s = 1; s <= 2 && K / 128 >= s; ++s) {
            if (((N + 63) / 64) * s < 192) continue;
            p.use = true;
            p.nb = 4;
            p.ksplit = s;
            p.krange = krange_of(s);
            return p;
        }
        return p;
    }
    if (lds) {
        // no register limit on the K range: the widest weight tile first, then
        // the fewest splits that give at least 192 workgroups
        for (int nb = 4; nb >= 2; nb -= 2)
            for (int s = 1; s <= 8 && K / 128 >= s; s *= 2) {
                if (((N + 16 * nb - 1) / (16 * nb)) * s < 192) continue;
                p.use = true;
                p.nb = nb;
                p.ksplit = s;
                p.krange = krange_of(s);
                return p;
            }
        return p;
    }
    const int maxch = stream_max_chunks(am, p.mb);
    // the fewest K splits (partial sums cost an extra pass) that fit the
    // activation registers and give at least 192 workgroups, wider weight
    // tiles first (measured: 192-768 resident workgroups stream alike)
    for (int s = 1; s <= 8; s *= 2) {
        if (K / 128 < s) break;
        const int64_t krange = krange_of(s);
        const int64_t chunks = (krange + 1023) / 1024;
        int nch = 1;
        while (nch < chunks) nch *= 2;
        if (nch > maxch) continue;
        for (int nb = 4; nb >= 2; nb -= 2) {
            if (((N + 16 * nb - 1) / (16 * nb)) * s < 192) continue;
            p.use = true;
            p.nb = nb;
            p.ksplit = s;
            p.krange = krange;
            return p;
        }
    }
    return p;
}

hipError_t run_stream(const StreamPlan& p, const void* a, const uint8_t* a_scales, const float* a_global,
                      int64_t M, int64_t N, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                      const float* w_global, uint16_t* y, float* partial, hipStream_t s) {
    StreamArgs g;
    g.a = a;
    g.a_scales = a_scales;
    g.a_global = a_global;
    g.b_codes = w_codes;
    g.b_scales = w_scales;
    g.b_global = w_global;
    g.M = M;
    g.N = N;
    g.K = K;
    g.ksplit = p.ksplit;
    g.krange = p.krange;
    g.out = p.ksplit > 1 ? static_cast<void*>(partial) : static_cast<void*>(y);
    hipError_t e = launch_gemm_stream(g, p.am, p.nb, p.mb, s);
    if (e != hipSuccess || p.ksplit == 1) return e;
    return launch_splitk_reduce(partial, p.ksplit, M, N, w_global, a_global, y, s);
}

size_t stream_partial_bytes(const StreamPlan& p, int64_t M, int64_t N) {
    return p.use && p.ksplit > 1 ? align_up((size_t)p.ksplit * (size_t)(M * N) * 4) : 0;
}

// Rows of the activation handled per GEMM launch: the kernel addresses the
// decoded activation through one buffer resource, which spans < 2 GiB.
int64_t gemm_chunk_rows(int64_t M, int64_t K) {
    int64_t cap = (kMaxOperandBytes - 1) / (K * 2);
    if (cap >= 256) cap = cap / 256 * 256;
    return cap < M ? cap : M;
}

struct GemmLayout {
    size_t xhat = 0, partial = 0, total = 0;
};

// W4A4 workspace: the quantized activation (exact f16 q * s for the tiles,
// bf16 for the GEMV, packed codes and scales for the stream kernel) and the
// split-K partial sums of whichever kernel the plans pick.
GemmLayout layout_gemm(int64_t M, int64_t N, int64_t K) {
    GemmLayout l;
    const GemmPlan p = plan_gemm(M, N, K);
    const StreamPlan sp = plan_stream(M, N, K, SAct::kPacked);
    const StreamPlan sq = plan_stream(M, N, K, SAct::kQuant);
    size_t off = 0;
    l.xhat = off; off += align_up((size_t)(M * K * 2));
    size_t part = 0;
    if (sp.use || sq.use) {
        part = std::max(stream_partial_bytes(sp, M, N), stream_partial_bytes(sq, M, N));
    } else if (!p.gemv && p.ksplit > 1) {
        part = align_up((size_t)p.ksplit * (size_t)(gemm_chunk_rows(M, K) * N) * 4);
    }
    if (part) {
        l.partial = off;
        off += part;
    }
    l.total = off;
    return l;
}

// W4A16 GEMM workspace: split-K partial sums only (the activation is the
// bf16 operand itself).
GemmLayout layout_gemm_w4a16(int64_t M, int64_t N, int64_t K) {
    GemmLayout l;
    const GemmPlan p = plan_gemm(M, N, K, true);
    const StreamPlan sp = plan_stream(M, N, K, SAct::kBf16);
    if (sp.use) l.total = stream_partial_bytes(sp, M, N);
    else if (!p.gemv && p.ksplit > 1) l.total = align_up((size_t)p.ksplit * (size_t)(gemm_chunk_rows(M, K) * N) * 4);
    l.partial = 0;
    return l;
}

// The MFMA-tile path shared by both GEMMs: A is a 16-bit [M, K] operand (f16
// q * s for W4A4, the bf16 activation for W4A16), in launches of at most
// gemm_chunk_rows rows; split K reduces through `partial`.
hipError_t run_gemm_tiles(const GemmPlan& p, const uint16_t* a, AFmt afmt, const float* a_global, int64_t M,
                          int64_t N, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                          const float* w_global, uint16_t* y, float* partial, hipStream_t s) {
    const int64_t chunk = gemm_chunk_rows(M, K);
    for (int64_t r0 = 0; r0 < M; r0 += chunk) {
        const int64_t rows = (M - r0 < chunk) ? M - r0 : chunk;
        GemmArgs g;
        g.a = a + r0 * K;
        g.a_src_rows = rows;
        g.a_global = a_global;
        g.b_codes = w_codes;
        g.b_scales = w_scales;
        g.b_global = w_global;
        g.M = rows;
        g.N = N;
        g.K = K;
        g.ksplit = p.ksplit;
        hipError_t e;
        if (p.sk_wgs > 0) {
            g.ksplit = 1;
            g.sk_wgs = p.sk_wgs;
            g.sk_y = y + r0 * N;
            g.out = partial;
            g.ldo = N;
            e = launch_gemm_a16(g, afmt, Epi::kPartialF32, p.tile, 0, s);
            if (e != hipSuccess) return e;
            e = launch_streamk_reduce(partial, rows, N, K, p.tile, p.sk_wgs, w_global, a_global, y + r0 * N, s);
        } else if (p.ksplit > 1) {
            g.out = partial;
            g.ldo = N;
            e = launch_gemm_a16(g, afmt, Epi::kPartialF32, p.tile, 0, s);
            if (e != hipSuccess) return e;
            e = launch_splitk_reduce(partial, p.ksplit, rows, N, w_global, a_global, y + r0 * N, s);
        } else {
            g.out = y + r0 * N;
            g.ldo = N;
            e = launch_gemm_a16(g, afmt, Epi::kStoreBf16, p.tile, 0, s);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------------ MoE planning --

// Row tile of the grouped GEMMs: a group's rows are covered by tiles of this
// height, multiplied by four waves of 96 x 64 (a tile of at most 128 rows
// splits them 64 / 64 between its wave rows).  With about 128 rows per
// expert, 128-row tiles give half the experts a second tile of a few rows
// that still loads and decodes the expert's whole weight tile (with every
// expert at exactly 128 rows the layer took 3.4 ms against 4.2 ms on the
// benchmark's routing of 103-157 rows); 192-row tiles hold every such
// expert in one (measured on MI355X, benchmark routing, random NVFP4
// experts: W4A16 4.21-4.44 -> 3.78-3.88 ms, W4A4 4.10-4.25 -> 3.78 ms,
// bit-identical; with every expert at exactly 128 rows 3.39 / 3.30 ->
// 3.62 / 3.80 ms).  Earlier 192-row tiles of six 64 x 64 waves decoded each
// weight tile three times and lost (5.3 ms).
constexpr int kMoeBM = 192;

struct MoeLayout {
    size_t row_off = 0, tile_off = 0, perm = 0, inv = 0, pos_group = 0, route = 0;
    size_t xq = 0, hq = 0, h = 0, y = 0, z13 = 0, z2 = 0, shared = 0, total = 0;
};

// lora_rank > 0 adds the bf16 rank-r projections z13 [T, r] and z2 [S, r].
MoeLayout layout_moe(const nvfp4_moe_problem& p, int64_t lora_rank = 0) {
    MoeLayout l;
    const size_t S = (size_t)(p.T * p.top_k);
    size_t off = 0;
    l.row_off = off; off += align_up((size_t)(p.E + 1) * 4);
    l.tile_off = off; off += align_up((size_t)(p.E + 1) * 4);
    l.perm = off; off += align_up(S * 4);
    l.inv = off; off += align_up(S * 4);
    l.pos_group = off; off += align_up(S * 4);
    l.route = off; off += align_up(moe_route_scratch_bytes((int64_t)S, (int32_t)p.E));
    if (p.mode == 1) {
        // the quantized activations as exact f16 products q * s, slot order
        // (token order when every expert shares one a13 value), and that choice
        l.xq = off; off += align_up(S * (size_t)p.H * 2);
        l.hq = off; off += align_up(S * (size_t)p.I * 2);
        l.shared = off; off += align_up(4);
    }
    l.h = off; off += align_up(S * (size_t)p.I * 2);
    l.y = off; off += align_up(S * (size_t)p.H * 4);
    if (lora_rank > 0) {
        l.z13 = off; off += align_up((size_t)p.T * (size_t)lora_rank * 2);
        l.z2 = off; off += align_up(S * (size_t)lora_rank * 2);
    }
    l.total = off;
    return l;
}

template <typename T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

int32_t nvfp4_version(void) { return 100; }

const char* nvfp4_status_string(int32_t status) {
    switch (status) {
        case NVFP4_OK: return "ok";
        case NVFP4_ERR_NULL_ARG: return "null argument";
        case NVFP4_ERR_SHAPE: return "invalid shape";
        case NVFP4_ERR_ALIGN: return "misaligned pointer";
        case NVFP4_ERR_UNSUPPORTED: return "unsupported problem";
        case NVFP4_ERR_WORKSPACE: return "workspace too small";
        case NVFP4_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* nvfp4_last_error(void) { return g_last_error; }

// ---------------------------------------------------------------- quantize --

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return align_up((size_t)amax_grid(rows * cols) * 4);
}

int32_t nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, const float* static_scale,
                       uint8_t* codes, uint8_t* scales, float* global_scale, void* workspace,
                       size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (rows < 0 || cols <= 0 || cols % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "quantize: need rows >= 0, cols > 0 and cols %% 16 == 0%s");
    if (rows == 0) return NVFP4_OK;
    if (!x || !codes || !scales || !global_scale)
        return fail(NVFP4_ERR_NULL_ARG, "quantize: x, codes, scales and global_scale are required%s");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned4(global_scale) ||
        (static_scale && !aligned4(static_scale)) || (workspace && !aligned16(workspace)))
        return fail(NVFP4_ERR_ALIGN, "quantize: pointers must be 16-byte aligned%s");
    const size_t need = static_scale ? 0 : nvfp4_quantize_workspace_size(rows, cols);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(NVFP4_ERR_WORKSPACE, "quantize: dynamic mode needs nvfp4_quantize_workspace_size bytes%s");
    hipStream_t s = as_stream(stream);
    PackArgs a;
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.codes = codes;
    a.scales = scales;
    a.global_out = global_scale;
    if (static_scale) {
        a.mode = ScaleMode::kStatic;
        a.sg_ptr = static_scale;
    } else {
        const int grid = amax_grid(rows * cols);
        uint32_t* partial = reinterpret_cast<uint32_t*>(workspace);
        int32_t st = hip_status(launch_amax_partial(x, rows * cols, partial, grid, s), "quantize amax");
        if (st) return st;
        a.mode = ScaleMode::kDynamic;
        a.partial = partial;
        a.npartial = grid;
    }
    return hip_status(launch_quantize_pack(a, s), "quantize pack");
}

int32_t nvfp4_quantize_noalloc(const uint16_t* x, int64_t rows, int64_t cols, const float* static_scale,
                               uint8_t* codes, uint8_t* scales, float* global_scale, void* stream) {
    g_last_error[0] = '\0';
    if (rows < 0 || cols <= 0 || cols % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "quantize_noalloc: need rows >= 0, cols > 0 and cols %% 16 == 0%s");
    if (rows > ((int64_t)1 << 62) / cols)
        return fail(NVFP4_ERR_UNSUPPORTED, "quantize_noalloc: rows * cols overflows%s");
    if (!static_scale && amax_grid(rows * cols) > kNoAllocPartials)
        return fail(NVFP4_ERR_UNSUPPORTED, "quantize_noalloc: more partial maxima than the static scratch holds%s");
    if (rows == 0) return NVFP4_OK;
    if (!x || !codes || !scales || !global_scale)
        return fail(NVFP4_ERR_NULL_ARG, "quantize_noalloc: x, codes, scales and global_scale are required%s");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned4(global_scale) ||
        (static_scale && !aligned4(static_scale)))
        return fail(NVFP4_ERR_ALIGN, "quantize_noalloc: pointers must be 16-byte aligned%s");
    hipStream_t s = as_stream(stream);
    if (static_scale)   // one pass, no scratch
        return nvfp4_quantize(x, rows, cols, static_scale, codes, scales, global_scale, nullptr, 0, stream);
    uint32_t* partial = nullptr;
    int32_t st = hip_status(noalloc_partials(s, &partial), "quantize_noalloc scratch");
    if (st) return st;
    return nvfp4_quantize(x, rows, cols, nullptr, codes, scales, global_scale, partial,
                          (size_t)kNoAllocPartials * sizeof(uint32_t), stream);
}

int32_t nvfp4_quantize_columnwise(const uint16_t* x, int64_t rows, int64_t cols, const float* static_scale,
                                  uint8_t* codes_t, uint8_t* scales_t, float* global_scale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (rows < 0 || cols < 0 || rows % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "quantize_columnwise: need rows, cols >= 0 and rows %% 16 == 0%s");
    if (cols % 8 != 0) return fail(NVFP4_ERR_UNSUPPORTED, "quantize_columnwise: cols must be a multiple of 8%s");
    if ((rows + 127) / 128 > 65535)
        return fail(NVFP4_ERR_UNSUPPORTED, "quantize_columnwise: at most 65535 x 128 rows%s");
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!x || !codes_t || !scales_t || !global_scale)
        return fail(NVFP4_ERR_NULL_ARG, "quantize_columnwise: x, codes, scales and global_scale are required%s");
    if (!aligned16(x) || !aligned16(codes_t) || !aligned16(scales_t) || !aligned4(global_scale) ||
        (static_scale && !aligned4(static_scale)) || (workspace && !aligned16(workspace)))
        return fail(NVFP4_ERR_ALIGN, "quantize_columnwise: pointers must be 16-byte aligned%s");
    const size_t need = static_scale ? 0 : nvfp4_quantize_workspace_size(rows, cols);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(NVFP4_ERR_WORKSPACE, "quantize_columnwise: dynamic mode needs nvfp4_quantize_workspace_size bytes%s");
    hipStream_t s = as_stream(stream);
    if (static_scale)
        return hip_status(launch_quantize_cols(x, rows, cols, ScaleMode::kStatic, nullptr, 0, static_scale, codes_t,
                                               scales_t, global_scale, s),
                          "quantize_columnwise");
    const int grid = amax_grid(rows * cols);
    uint32_t* partial = reinterpret_cast<uint32_t*>(workspace);
    int32_t st = hip_status(launch_amax_partial(x, rows * cols, partial, grid, s), "quantize_columnwise amax");
    if (st) return st;
    return hip_status(launch_quantize_cols(x, rows, cols, ScaleMode::kDynamic, partial, grid, nullptr, codes_t,
                                           scales_t, global_scale, s),
                      "quantize_columnwise");
}

int32_t nvfp4_dequantize_transpose(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                                   int64_t rows, int64_t cols, uint16_t* y_t, void* stream) {
    g_last_error[0] = '\0';
    if (rows < 0 || cols <= 0 || cols % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "dequantize_transpose: need rows >= 0, cols > 0 and cols %% 16 == 0%s");
    if (rows % 8 != 0) return fail(NVFP4_ERR_UNSUPPORTED, "dequantize_transpose: rows must be a multiple of 8%s");
    if ((cols + 127) / 128 > 65535)
        return fail(NVFP4_ERR_UNSUPPORTED, "dequantize_transpose: at most 65535 x 128 cols%s");
    if (rows == 0) return NVFP4_OK;
    if (!codes || !scales || !global_scale || !y_t)
        return fail(NVFP4_ERR_NULL_ARG, "dequantize_transpose: all pointers are required%s");
    if (!aligned16(codes) || !aligned16(scales) || !aligned4(global_scale) || !aligned16(y_t))
        return fail(NVFP4_ERR_ALIGN, "dequantize_transpose: pointers must be 16-byte aligned%s");
    return hip_status(launch_dequantize_t(codes, scales, global_scale, rows, cols, y_t, as_stream(stream)),
                      "dequantize_transpose");
}

int32_t nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                         int64_t rows, int64_t cols, uint16_t* y, void* stream) {
    g_last_error[0] = '\0';
    if (rows < 0 || cols <= 0 || cols % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "dequantize: need rows >= 0, cols > 0 and cols %% 16 == 0%s");
    if (rows == 0) return NVFP4_OK;
    if (!codes || !scales || !global_scale || !y)
        return fail(NVFP4_ERR_NULL_ARG, "dequantize: all pointers are required%s");
    if (!aligned16(codes) || !aligned16(scales) || !aligned4(global_scale) || !aligned16(y))
        return fail(NVFP4_ERR_ALIGN, "dequantize: pointers must be 16-byte aligned%s");
    return hip_status(launch_dequantize(codes, scales, global_scale, 0.0f, rows, cols, y, as_stream(stream)),
                      "dequantize");
}

// -------------------------------------------------------------------- GEMV --

int32_t nvfp4_gemv_w4a16(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_codes,
                         const uint8_t* w_scales, const float* w_global, uint16_t* y, void* stream) {
    g_last_error[0] = '\0';
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "gemv: need M, N >= 0, K > 0 and K %% 16 == 0%s");
    if (M > 8) return fail(NVFP4_ERR_UNSUPPORTED, "gemv: M must be <= 8%s");
    if (K % 32 != 0) return fail(NVFP4_ERR_UNSUPPORTED, "gemv: K must be a multiple of 32%s");
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!x || !w_codes || !w_scales || !w_global || !y)
        return fail(NVFP4_ERR_NULL_ARG, "gemv: all pointers are required%s");
    if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned4(w_global) || !aligned16(y))
        return fail(NVFP4_ERR_ALIGN, "gemv: pointers must be 16-byte aligned%s");
    // the stream kernel when it needs no K split (so no workspace): short
    // rows from M = 3, long rows from M = 5 (the activation through LDS)
    const StreamPlan sp = plan_stream(M, N, K, SAct::kBf16);
    if (sp.use && sp.ksplit == 1)
        return hip_status(run_stream(sp, x, nullptr, nullptr, M, N, K, w_codes, w_scales, w_global, y,
                                     nullptr, as_stream(stream)),
                          "gemv stream");
    return hip_status(launch_gemv_w4a16(x, (int)M, N, K, w_codes, w_scales, w_global, nullptr, y,
                                        as_stream(stream)),
                      "gemv");
}

// -------------------------------------------------------------------- GEMM --

size_t nvfp4_gemm_w4a4_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return 0;
    return layout_gemm(M, N, K).total;
}

int32_t nvfp4_gemm_w4a4(const uint16_t* x, const float* input_scale, int64_t M, int64_t N, int64_t K,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                        uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "gemm: need M, N >= 0, K > 0 and K %% 16 == 0%s");
    if (K % 64 != 0) return fail(NVFP4_ERR_UNSUPPORTED, "gemm: K must be a multiple of 64%s");
    if (!plan_gemm(M, N, K).gemv && ((int64_t)N * (K / 2) >= kMaxOperandBytes || gemm_chunk_rows(M, K) < 1))
        return fail(NVFP4_ERR_UNSUPPORTED, "gemm: weight matrix of 2 GiB or more%s");
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!x || !input_scale || !w_codes || !w_scales || !w_global || !y)
        return fail(NVFP4_ERR_NULL_ARG, "gemm: x, input_scale, weights and y are required%s");
    if (!aligned16(x) || !aligned4(input_scale) || !aligned16(w_codes) || !aligned16(w_scales) ||
        !aligned4(w_global) || !aligned16(y) || (workspace && !aligned16(workspace)))
        return fail(NVFP4_ERR_ALIGN, "gemm: pointers must be 16-byte aligned%s");
    const GemmLayout l = layout_gemm(M, N, K);
    if (!workspace || workspace_bytes < l.total)
        return fail(NVFP4_ERR_WORKSPACE, "gemm: workspace smaller than nvfp4_gemm_w4a4_workspace_size%s");
    hipStream_t s = as_stream(stream);
    // Up to M = 16 on short rows the stream kernel quantizes the activation
    // in registers, one launch (measured on MI355X, q_b_proj 16384 x 2048:
    // M = 8 12.1 -> 10.2 us, M = 16 12.1 -> 11.0 us against the separate
    // quantize launch); beyond that the redundant encode in every workgroup
    // costs more than that launch (M = 32 15.1 against 13.8 us).
    const StreamPlan sq = plan_stream(M, N, K, SAct::kQuant);
    if (sq.use && M <= 16 && K <= 4096)
        return hip_status(run_stream(sq, x, nullptr, input_scale, M, N, K, w_codes, w_scales, w_global,
                                     y, sq.ksplit > 1 ? at<float>(workspace, l.partial) : nullptr, s),
                          "gemm stream");
    const StreamPlan sp = plan_stream(M, N, K, SAct::kPacked);
    if (sp.use) {
        // the static quantize writes the packed activation (codes, then scale
        // bytes) into the workspace; the stream kernel decodes it in registers
        uint8_t* ac = at<uint8_t>(workspace, l.xhat);
        uint8_t* as = ac + align_up((size_t)(M * K / 2));
        PackArgs a;
        a.x = x;
        a.rows = M;
        a.cols = K;
        a.mode = ScaleMode::kStatic;
        a.sg_ptr = input_scale;
        a.codes = ac;
        a.scales = as;
        int32_t st = hip_status(launch_quantize_pack(a, s), "gemm activation quantize");
        if (st) return st;
        return hip_status(run_stream(sp, ac, as, input_scale, M, N, K, w_codes, w_scales, w_global, y,
                                     sp.ksplit > 1 ? at<float>(workspace, l.partial) : nullptr, s),
                          "gemm stream");
    }
    const GemmPlan p = plan_gemm(M, N, K);
    if (p.gemv && gemv_quantizes_activation((int)M, K))
        return hip_status(launch_gemv_w4a4(x, (int)M, N, K, w_codes, w_scales, w_global, input_scale, y, s),
                          "gemm gemv");
    // Static activation quantization under input_scale.  The GEMM consumes the
    // quantized activation as the exact products q * s (f16 for the MFMA path,
    // bf16 for the GEMV), written directly by the quantizer; the two global
    // scales are applied after the contraction.
    uint16_t* xh = at<uint16_t>(workspace, l.xhat);
    PackArgs a;
    a.x = x;
    a.rows = M;
    a.cols = K;
    a.mode = ScaleMode::kStatic;
    a.sg_ptr = input_scale;
    a.xhat = xh;
    a.xhat_bf16 = p.gemv;
    int32_t st = hip_status(launch_quantize_pack(a, s), "gemm activation quantize");
    if (st) return st;
    if (p.gemv)
        return hip_status(launch_gemv_w4a16(xh, (int)M, N, K, w_codes, w_scales, w_global, input_scale, y, s),
                          "gemm gemv");
    return hip_status(run_gemm_tiles(p, xh, AFmt::kF16, input_scale, M, N, K, w_codes, w_scales, w_global, y,
                                     p.ksplit > 1 ? at<float>(workspace, l.partial) : nullptr, s),
                      "gemm");
}

size_t nvfp4_gemm_w4a4_packed_workspace_size(int64_t M, int64_t N, int64_t K) {
    return nvfp4_gemm_w4a4_workspace_size(M, N, K);
}

int32_t nvfp4_gemm_w4a4_packed(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global, int64_t M,
                               int64_t N, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                               const float* w_global, uint16_t* y, void* workspace, size_t workspace_bytes,
                               void* stream) {
    g_last_error[0] = '\0';
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "gemm_packed: need M, N >= 0, K > 0 and K %% 16 == 0%s");
    if (K % 64 != 0) return fail(NVFP4_ERR_UNSUPPORTED, "gemm_packed: K must be a multiple of 64%s");
    if (!plan_gemm(M, N, K).gemv && ((int64_t)N * (K / 2) >= kMaxOperandBytes || gemm_chunk_rows(M, K) < 1))
        return fail(NVFP4_ERR_UNSUPPORTED, "gemm_packed: weight matrix of 2 GiB or more%s");
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!a_codes || !a_scales || !a_global || !w_codes || !w_scales || !w_global || !y)
        return fail(NVFP4_ERR_NULL_ARG, "gemm_packed: activation, weights and y are required%s");
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned4(a_global) || !aligned16(w_codes) ||
        !aligned16(w_scales) || !aligned4(w_global) || !aligned16(y) || (workspace && !aligned16(workspace)))
        return fail(NVFP4_ERR_ALIGN, "gemm_packed: pointers must be 16-byte aligned%s");
    const GemmLayout l = layout_gemm(M, N, K);
    if (!workspace || workspace_bytes < l.total)
        return fail(NVFP4_ERR_WORKSPACE, "gemm_packed: workspace smaller than nvfp4_gemm_w4a4_packed_workspace_size%s");
    hipStream_t s = as_stream(stream);
    const StreamPlan sp = plan_stream(M, N, K, SAct::kPacked);
    if (sp.use)
        return hip_status(run_stream(sp, a_codes, a_scales, a_global, M, N, K, w_codes, w_scales,
                                     w_global, y, sp.ksplit > 1 ? at<float>(workspace, l.partial) : nullptr, s),
                          "gemm_packed stream");
    const GemmPlan p = plan_gemm(M, N, K);
    // Small M on the fixed GEMV layouts: the GEMV decodes the packed
    // activation itself (one launch).
    if (p.gemv && gemv_takes_packed((int)M, K))
        return hip_status(launch_gemv_w4a4_packed(a_codes, a_scales, (int)M, N, K, w_codes, w_scales, w_global,
                                                  a_global, y, s),
                          "gemm_packed gemv");
    // Otherwise the packed activation is expanded to its exact products q * s, the
    // operand form of both kernels (bf16 for the GEMV, f16 for the tiles);
    // the two global scales are applied after the contraction.
    uint16_t* xh = at<uint16_t>(workspace, l.xhat);
    int32_t st = hip_status(launch_expand_qs(a_codes, a_scales, M, K, xh, p.gemv, s), "gemm_packed expand");
    if (st) return st;
    if (p.gemv)
        return hip_status(launch_gemv_w4a16(xh, (int)M, N, K, w_codes, w_scales, w_global, a_global, y, s),
                          "gemm_packed gemv");
    return hip_status(run_gemm_tiles(p, xh, AFmt::kF16, a_global, M, N, K, w_codes, w_scales, w_global, y,
                                     p.ksplit > 1 ? at<float>(workspace, l.partial) : nullptr, s),
                      "gemm_packed");
}

size_t nvfp4_gemm_w4a16_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return 0;
    return layout_gemm_w4a16(M, N, K).total;
}

int32_t nvfp4_gemm_w4a16(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w_codes,
                         const uint8_t* w_scales, const float* w_global, uint16_t* y, void* workspace,
                         size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0)
        return fail(NVFP4_ERR_SHAPE, "gemm_w4a16: need M, N >= 0, K > 0 and K %% 16 == 0%s");
    if (K % 64 != 0) return fail(NVFP4_ERR_UNSUPPORTED, "gemm_w4a16: K must be a multiple of 64%s");
    if (!plan_gemm(M, N, K, true).gemv && ((int64_t)N * (K / 2) >= kMaxOperandBytes || gemm_chunk_rows(M, K) < 1))
        return fail(NVFP4_ERR_UNSUPPORTED, "gemm_w4a16: weight matrix of 2 GiB or more%s");
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!x || !w_codes || !w_scales || !w_global || !y)
        return fail(NVFP4_ERR_NULL_ARG, "gemm_w4a16: x, weights and y are required%s");
    if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned4(w_global) || !aligned16(y) ||
        (workspace && !aligned16(workspace)))
        return fail(NVFP4_ERR_ALIGN, "gemm_w4a16: pointers must be 16-byte aligned%s");
    const GemmLayout l = layout_gemm_w4a16(M, N, K);
    if (l.total > 0 && (!workspace || workspace_bytes < l.total))
        return fail(NVFP4_ERR_WORKSPACE, "gemm_w4a16: workspace smaller than nvfp4_gemm_w4a16_workspace_size%s");
    hipStream_t s = as_stream(stream);
    const StreamPlan sp = plan_stream(M, N, K, SAct::kBf16);
    if (sp.use)
        return hip_status(run_stream(sp, x, nullptr, nullptr, M, N, K, w_codes, w_scales, w_global, y,
                                     sp.ksplit > 1 ? static_cast<float*>(workspace) : nullptr, s),
                          "gemm_w4a16 stream");
    const GemmPlan p = plan_gemm(M, N, K, true);
    if (p.gemv)
        return hip_status(launch_gemv_w4a16(x, (int)M, N, K, w_codes, w_scales, w_global, nullptr, y, s),
                          "gemm_w4a16 gemv");
    return hip_status(run_gemm_tiles(p, x, AFmt::kBf16, nullptr, M, N, K, w_codes, w_scales, w_global, y,
                                     p.ksplit > 1 ? at<float>(workspace, l.partial) : nullptr, s),
                      "gemm_w4a16");
}

// --------------------------------------------------------------------- MoE --

size_t nvfp4_moe_workspace_size(const nvfp4_moe_problem* p) {
    if (!p || p->T < 0 || p->E <= 0 || p->top_k <= 0 || p->H <= 0 || p->I <= 0) return 0;
    return layout_moe(*p).total;
}

size_t nvfp4_moe_lora_workspace_size(const nvfp4_moe_problem* p, const nvfp4_moe_lora* lora) {
    if (!p || p->T < 0 || p->E <= 0 || p->top_k <= 0 || p->H <= 0 || p->I <= 0) return 0;
    if (lora && lora->rank <= 0) return 0;
    return layout_moe(*p, lora ? lora->rank : 0).total;
}

int32_t nvfp4_moe_grouped_gemm(const nvfp4_moe_problem* p, const nvfp4_moe_tensors* t, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return nvfp4_moe_grouped_gemm_lora(p, t, nullptr, workspace, workspace_bytes, stream);
}

int32_t nvfp4_moe_grouped_gemm_lora(const nvfp4_moe_problem* p, const nvfp4_moe_tensors* t,
                                    const nvfp4_moe_lora* lora, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    g_last_error[0] = '\0';
    if (!p || !t) return fail(NVFP4_ERR_NULL_ARG, "moe: problem and tensors are required%s");
    if (p->T < 0 || p->E <= 0 || p->top_k <= 0 || p->H <= 0 || p->I <= 0 || p->H % 16 || p->I % 16 ||
        (p->mode != 0 && p->mode != 1))
        return fail(NVFP4_ERR_SHAPE, "moe: need T >= 0, E, top_k, H, I > 0, H and I multiples of 16, mode 0 or 1%s");
    if (p->H % 64 || p->I % 64) return fail(NVFP4_ERR_UNSUPPORTED, "moe: H and I must be multiples of 64%s");
    if (p->E > 4096) return fail(NVFP4_ERR_UNSUPPORTED, "moe: at most 4096 experts%s");
    if (p->T * p->top_k > (int64_t)1 << 30) return fail(NVFP4_ERR_UNSUPPORTED, "moe: too many slots%s");
    if (lora) {
        if (lora->rank <= 0) return fail(NVFP4_ERR_SHAPE, "moe lora: rank must be positive%s");
        if (lora->rank % 8 || lora->rank > 128)
            return fail(NVFP4_ERR_UNSUPPORTED, "moe lora: rank must be a multiple of 8 and at most 128%s");
    }
    {
        // the GEMM kernels address each operand through one buffer resource
        const int64_t S = p->T * p->top_k;
        const int64_t act = p->mode == 1 ? S * p->H * 2 : p->T * p->H * 2;
        if (act >= kMaxOperandBytes || S * p->I * 2 >= kMaxOperandBytes || 2 * p->I * (p->H / 2) >= kMaxOperandBytes ||
            p->H * (p->I / 2) >= kMaxOperandBytes)
            return fail(NVFP4_ERR_UNSUPPORTED, "moe: an operand of 2 GiB or more%s");
    }
    if (p->T == 0) return NVFP4_OK;
    if (!t->x || !t->topk_ids || !t->topk_weights || !t->w13_codes || !t->w13_scales || !t->w13_global ||
        !t->w2_codes || !t->w2_scales || !t->w2_global || !t->out ||
        (p->mode == 1 && (!t->a13_scale || !t->a2_scale)))
        return fail(NVFP4_ERR_NULL_ARG, "moe: a required tensor is NULL%s");
    const void* tensors[] = {t->x, t->w13_codes, t->w13_scales, t->w2_codes, t->w2_scales, t->out};
    for (const void* q : tensors)
        if (!aligned16(q)) return fail(NVFP4_ERR_ALIGN, "moe: tensor pointers must be 16-byte aligned%s");
    const void* words[] = {t->topk_ids, t->topk_weights, t->w13_global, t->w2_global};
    for (const void* q : words)
        if (!aligned4(q)) return fail(NVFP4_ERR_ALIGN, "moe: fp32/int32 arrays must be 4-byte aligned%s");
    if (p->mode == 1 && (!aligned4(t->a13_scale) || !aligned4(t->a2_scale)))
        return fail(NVFP4_ERR_ALIGN, "moe: fp32/int32 arrays must be 4-byte aligned%s");
    const bool lora13 = lora && (lora->a13 || lora->b13), lora2 = lora && (lora->a2 || lora->b2);
    if (lora && ((lora13 && (!lora->a13 || !lora->b13)) || (lora2 && (!lora->a2 || !lora->b2))))
        return fail(NVFP4_ERR_NULL_ARG, "moe lora: a13/b13 and a2/b2 are given in pairs%s");
    if (lora) {
        const void* adapters[] = {lora->a13, lora->b13, lora->a2, lora->b2};
        for (const void* q : adapters)
            if (q && !aligned16(q)) return fail(NVFP4_ERR_ALIGN, "moe lora: adapter tensors must be 16-byte aligned%s");
    }
    if (workspace && !aligned16(workspace)) return fail(NVFP4_ERR_ALIGN, "moe: workspace must be 16-byte aligned%s");
    const MoeLayout l = layout_moe(*p, lora ? lora->rank : 0);
    if (!workspace || workspace_bytes < l.total)
        return fail(NVFP4_ERR_WORKSPACE, lora ? "moe: workspace smaller than nvfp4_moe_lora_workspace_size%s"
                                              : "moe: workspace smaller than nvfp4_moe_workspace_size%s");

    hipStream_t s = as_stream(stream);
    const int64_t S = p->T * p->top_k;
    const int32_t E = (int32_t)p->E;
    int32_t* row_off = at<int32_t>(workspace, l.row_off);
    int32_t* tile_off = at<int32_t>(workspace, l.tile_off);
    int32_t* perm = at<int32_t>(workspace, l.perm);
    int32_t* inv = at<int32_t>(workspace, l.inv);
    int32_t* pos_group = at<int32_t>(workspace, l.pos_group);
    uint16_t* h = at<uint16_t>(workspace, l.h);
    float* Y = at<float>(workspace, l.y);
    int32_t st = hip_status(launch_moe_route(t->topk_ids, S, E, kMoeBM, row_off, tile_off, perm, inv, pos_group,
                                             at<int32_t>(workspace, l.route), s),
                            "moe route");
    if (st) return st;
    const int grid_m = (int)((S + kMoeBM - 1) / kMoeBM + E);

    // GEMM 1: [g | u] = x^ W13^T, h = bf16(silu(g) * u).  W4A16 multiplies the
    // bf16 tokens (gathered by slot); W4A4 first quantizes them per expert
    // group under a13_scale into their exact f16 products q * s, one row per
    // slot, or, when all E values of a13_scale are bitwise equal (the serving
    // form with one input scale for the experts' gate/up projections), one
    // row per token, which GEMM 1 then gathers by slot like the bf16 tokens:
    // the same operand values from an eighth of the quantize work (the
    // quantize pass takes that choice on the device and leaves it in the
    // workspace for GEMM 1).
    const A16Tile tile = A16Tile::k192x128_w96x64;  // kMoeBM-row tiles, as the routing counted
    GemmArgs g1;
    g1.b_codes = t->w13_codes;
    g1.b_scales = t->w13_scales;
    g1.b_global = t->w13_global;
    g1.M = S;
    g1.N = 2 * p->I;
    g1.K = p->H;
    g1.row_off = row_off;
    g1.tile_off = tile_off;
    g1.groups = E;
    // W4A4: the gate/up epilogue quantizes h under a2_scale itself and writes
    // the down projection's operand (f16 q * s); the bf16 h is kept only for
    // the LoRA down projection's shared A, which reads it
    g1.out = (p->mode == 1 && !lora2) ? nullptr : h;
    g1.ldo = p->I;
    if (p->mode == 1) {
        g1.out_q = at<uint16_t>(workspace, l.hq);
        g1.q_global = t->a2_scale;
    }
    g1.half_n = p->I;
    AFmt af = AFmt::kBf16;
    if (p->mode == 1) {
        uint16_t* xq = at<uint16_t>(workspace, l.xq);
        PackArgs a;
        a.x = t->x;
        a.rows = S;
        a.cols = p->H;
        a.src_row = perm;
        a.src_div = (int32_t)p->top_k;
        a.rows_valid = row_off + E;
        a.mode = ScaleMode::kGrouped;
        a.sg_group = t->a13_scale;
        a.row_group = pos_group;
        a.xhat = xq;
        int32_t* shared = at<int32_t>(workspace, l.shared);
        a.n_groups = E;
        a.shared_rows = p->T;
        a.shared_out = shared;
        st = hip_status(launch_quantize_pack(a, s), "moe activation quantize");
        if (st) return st;
        g1.a = xq;
        g1.a_src_rows = S;
        g1.a_rows = perm;
        g1.a_div = (int32_t)p->top_k;
        g1.a_rows_on = shared;
        g1.a_global = t->a13_scale;
        af = AFmt::kF16;
    } else {
        g1.a = t->x;
        g1.a_rows = perm;
        g1.a_div = (int32_t)p->top_k;
        g1.a_src_rows = p->T;
    }
    if (lora13) {
        // LoRA on gate/up: z13 = bf16(x A13^T) per token; the epilogue adds
        // scale * z13[token] B13_e^T before the activation
        uint16_t* z13 = at<uint16_t>(workspace, l.z13);
        st = hip_status(launch_lora_a(t->x, p->T, p->H, lora->a13, (int)lora->rank, z13, s), "moe lora a13");
        if (st) return st;
        g1.lora_z = z13;
        g1.lora_rows = perm;
        g1.lora_div = (int32_t)p->top_k;
        g1.lora_b = lora->b13;
        g1.lora_rank = (int32_t)lora->rank;
        g1.lora_scale = lora->scale;
    }
    st = hip_status(launch_gemm_a16(g1, af, lora13 ? Epi::kMoeGateUpLora : Epi::kMoeGateUp, tile, grid_m, s),
                    "moe gemm1");
    if (st) return st;

    // GEMM 2: Y = h^ W2^T (fp32, per slot row)
    GemmArgs g2;
    g2.b_codes = t->w2_codes;
    g2.b_scales = t->w2_scales;
    g2.b_global = t->w2_global;
    g2.M = S;
    g2.N = p->H;
    g2.K = p->I;
    g2.row_off = row_off;
    g2.tile_off = tile_off;
    g2.groups = E;
    g2.out = Y;
    g2.ldo = p->H;
    g2.a_src_rows = S;
    if (p->mode == 1) {
        g2.a = at<uint16_t>(workspace, l.hq);   // written by GEMM 1's epilogue
        g2.a_global = t->a2_scale;
    } else {
        g2.a = h;
    }
    if (lora2) {
        // LoRA on down: z2 = bf16(h A2^T) per slot row (expert-sorted, like h)
        uint16_t* z2 = at<uint16_t>(workspace, l.z2);
        st = hip_status(launch_lora_a(h, S, p->I, lora->a2, (int)lora->rank, z2, s), "moe lora a2");
        if (st) return st;
        g2.lora_z = z2;
        g2.lora_b = lora->b2;
        g2.lora_rank = (int32_t)lora->rank;
        g2.lora_scale = lora->scale;
    }
    st = hip_status(launch_gemm_a16(g2, af, lora2 ? Epi::kMoeDownLora : Epi::kMoeDown, tile, grid_m, s),
                    "moe gemm2");
    if (st) return st;
    return hip_status(launch_moe_combine(Y, inv, t->topk_weights, p->T, (int32_t)p->top_k, p->H, t->out, s),
                      "moe combine");
}

}  // extern "C"
