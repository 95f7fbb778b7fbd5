// Kernel selection of libqbd: which kernel (and tile shape) serves a call of
// a given shape.  Pure integer rules, host side, with the CU count passed in,
// so that the rules can be checked on a machine without a GPU.
//
// The rules follow the shape-regime split of Lumen v0.4.0 release page,
// "Phase 7.P - per-shape hybrid dispatch" and the central arch + shape
// table of LSE v0.4.16 release page, "Combined M8 Q4 gate/up execution":
// the kernel depends on (M, N, K), the weight format and the CU count, and
// never on whether the call is the fused gate/up form.  The fp32-activation
// plan takes no mode argument at all; where a kernel's resources differ
// between one and two weight matrices, the budget is that of two, so a
// fused call and the unfused calls of the same shape run the same kernel
// family with the same per-output summation order.
#pragma once

#include <stdint.h>

namespace qbd {

enum class Fmt : int { Q8_0 = 0, Q4 = 1 };
enum class Mode : int { Plain = 0, SwiGLU = 1 };

namespace plan {

constexpr int64_t kLanes = 64;                 // wave64
constexpr int64_t kLdsBytes = 160 * 1024;      // LDS of one gfx950 workgroup
constexpr int64_t kMaxGridY = 65535;

constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
constexpr int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

// ------------------------------------------------------- fp32 activations
// codes per 16-byte weight chunk, and the most K sweeps (64 chunks each)
// whose activation slices stay in VGPRs at M = 1
constexpr int64_t chunk_codes(Fmt f) { return f == Fmt::Q8_0 ? 16 : 32; }
constexpr int64_t max_vgpr_sweeps(Fmt f) { return f == Fmt::Q8_0 ? 8 : 4; }
constexpr int64_t m1_sweeps(Fmt f, int64_t K) { return cdiv(K / chunk_codes(f), kLanes); }

// rows per workgroup of the one-workgroup-per-CU kernels
constexpr int64_t resident_rows(int64_t N, int64_t cus) {
    return cdiv(N, imax(1, imin(cus, cdiv(N, 16))));
}

// M = 1 with x staged in LDS: the staged x plus the workgroup's outputs
constexpr int64_t m1_staged_lds_bytes(Fmt f, int64_t K, int64_t rows) {
    return (m1_sweeps(f, K) * kLanes * chunk_codes(f) + rows) * 4;
}
// staging x pays once x (4K bytes) is large next to the weight bytes a
// wave streams per x load
constexpr bool m1_stage_x(Fmt f, int64_t N, int64_t K) {
    return K >= (f == Fmt::Q8_0 ? 4096 : 2048) && N >= 4096;
}
// M = 1 with at least 2 K sweeps and fewer rows than this: one wave per
// sweep (the per-row grid would leave most SIMDs with less than one wave),
// one row per workgroup, two from 512 rows (the x slice of a wave then
// serves two rows: the 896 x 4864 down projection 3.44-3.56 against
// 3.91 us, four rows 3.56-3.59 us).  Q8_0 up to 16
// sweeps; 4-bit rows only up to the sweeps the per-row kernel holds, since
// a 4-bit chunk meets 32 floats of x, and past that the kernel with x
// staged in LDS is faster.
constexpr int64_t kM1SweepMaxRows = 4096;
constexpr int64_t kM1SweepMaxJ = 16;
constexpr int64_t m1_sweep_max_j(Fmt f) { return f == Fmt::Q8_0 ? kM1SweepMaxJ : max_vgpr_sweeps(f); }
constexpr bool m1_sweep(Fmt f, int64_t N, int64_t K) {
    return m1_sweeps(f, K) >= 2 && m1_sweeps(f, K) <= m1_sweep_max_j(f) && N < kM1SweepMaxRows;
}
constexpr int64_t m1_sweep_rows(int64_t N) { return N >= 512 ? 2 : 1; }
// rows past which M = 1 runs on the persistent grid (16 workgroups per CU
// of two-row waves); the choice keeps the per-row arithmetic
constexpr int64_t kM1PipeMinRows = 4096 * 4 * 2;

// VALU panels (M >= 2): the panel staged in LDS in sweeps of 1024 columns
constexpr int64_t kPanelKC = 1024;
constexpr int64_t panel_sweeps(int64_t K) { return cdiv(K / 16, kLanes); }
constexpr int64_t resident_lds_bytes(int64_t mt, int64_t K, int64_t rows, bool ylds) {
    return (mt * panel_sweeps(K) * kPanelKC + (ylds ? mt * rows : 0)) * 4;
}
constexpr int64_t panel_rows(int64_t M) { return M <= 4 ? 4 : 8; }

// matrix-core panel (M = 2 .. 16): 8 waves, at most 6 tiles of 16 rows per
// workgroup (5 for 16-row panels, whose two-matrix form would not keep six
// tiles' accumulators in 256 VGPRs without spilling), LDS holding the tiles'
// scale rows and then the partial sums
constexpr int64_t kMfmaWaves = 8;
constexpr int64_t kMfmaMaxNT = 6;
constexpr int64_t mfma_max_nt(int64_t rows) { return rows == 16 ? 5 : kMfmaMaxNT; }
constexpr int64_t mfma_scale_row(int64_t nb) { return cdiv(nb, 4) * 4 + 4; }
constexpr int64_t mfma_lds_bytes(int64_t nw, int64_t nt, int64_t nmat, int64_t mto, int64_t nb) {
    return imax(nmat * nt * 16 * mfma_scale_row(nb) * 2, nw * nt * nmat * mto * 16 * 4);
}
constexpr int64_t mfma_rows(int64_t M) { return M <= 8 ? 8 : 16; }
constexpr int64_t mfma_nt(int64_t M, int64_t N, int64_t cus) {
    return imin(mfma_max_nt(mfma_rows(M)), cdiv(cdiv(N, 16), cus));
}
// Every wave needs a group of blocks, the tiles must spread over the CUs,
// and the scale rows of two weight matrices must fit in LDS (the budget of
// the fused form, whatever the call).
constexpr bool mfma_supported(Fmt f, int64_t M, int64_t N, int64_t K, int64_t cus) {
    return M >= 2 && M <= 16 && cdiv(K / 32, f == Fmt::Q4 ? 4 : 2) >= kMfmaWaves && cdiv(N, 16) >= cus &&
           mfma_lds_bytes(kMfmaWaves, mfma_nt(M, N, cus), 2, mfma_rows(M), K / 32) <= kLdsBytes;
}
// Measured against the VALU panels: the matrix cores win for panels of
// 9-16 rows (the VALU kernels take two passes of 8) and for 4-bit weights
// with at least two 16-row tiles per CU; int8 panels of up to 8 rows and
// short, wide 4-bit shapes stay on the VALU.
constexpr bool mfma_preferred(Fmt f, int64_t M, int64_t N, int64_t cus) {
    return M > 8 || (f == Fmt::Q4 && cdiv(N, 16) >= 2 * cus);
}

enum class F32Kernel : int {
    M1Vgpr = 0,     // M = 1, x in VGPRs (per-row grid, or persistent for many rows)
    M1Staged = 1,   // M = 1, x staged once per workgroup in LDS
    Generic = 2,    // any M, x from global memory (fallback)
    Mfma = 3,       // M = 2..16, bf16 matrix cores, exact 3-part split of x
    Resident = 4,   // M >= 2, whole panel in LDS
    Chunked = 5,    // M >= 2, panel streamed through LDS in chunks of K
    M1Sweep = 6,    // M = 1, long rows and few of them: one wave per K sweep
};

struct F32Plan {
    F32Kernel kernel;
    int64_t sweeps;  // M1Vgpr: K sweeps held in VGPRs
    int64_t mt;      // panel rows per pass (Resident, Chunked, Generic, Mfma)
    int64_t nt;      // Mfma: 16-row tiles per workgroup
};

constexpr F32Plan f32_plan(Fmt f, int64_t M, int64_t N, int64_t K, int64_t cus) {
    if (M == 1) {
        const int64_t J = m1_sweeps(f, K);
        if (m1_sweep(f, N, K)) return {F32Kernel::M1Sweep, J, 1, 0};
        const bool fits = m1_staged_lds_bytes(f, K, resident_rows(N, cus)) <= kLdsBytes;
        if (J <= max_vgpr_sweeps(f) && !(fits && m1_stage_x(f, N, K))) return {F32Kernel::M1Vgpr, J, 1, 0};
        if (fits) return {F32Kernel::M1Staged, J, 1, 0};
        return {F32Kernel::Generic, 0, 1, 0};
    }
    if (mfma_supported(f, M, N, K, cus) && mfma_preferred(f, M, N, cus))
        return {F32Kernel::Mfma, 0, mfma_rows(M), mfma_nt(M, N, cus)};
    const int64_t mt = panel_rows(M);
    // more row groups than a grid's y dimension holds: the generic kernel,
    // which loops over row groups
    if (cdiv(M, mt) > kMaxGridY) return {F32Kernel::Generic, 0, 4, 0};
    if (resident_lds_bytes(mt, K, resident_rows(N, cus), false) <= kLdsBytes)
        return {F32Kernel::Resident, 0, mt, 0};
    return {F32Kernel::Chunked, 0, mt, 0};
}

// ----------------------------------------------------- Q8 activations
enum class Q8Kernel : int {
    Dot4 = 0,       // M < 16: v_dot4_i32_i8, one output row per wave
    SplitK = 1,     // 16 <= M <= 64 with few output tiles: K split over a workgroup's waves
    Panel = 2,      // otherwise: 32 x 32 int8 MFMA tiles per wave
    Tile16 = 3,     // short panels (Q8_0 8..64 rows, 4-bit 8..16): one 16 x 16 int8 tile per workgroup
    M1Staged = 4,   // M = 1: the activation panel staged in LDS once per workgroup
    PanelStaged = 5,  // 2 <= M <= 8: the panel staged in LDS step by step, each weight row read once
    Tile16Persist = 6,  // 8 <= M <= 16 over many tiles: one 8-wave workgroup per CU walks the tiles
};

constexpr int64_t kMfmaMinRows = 16;
constexpr int64_t kSplitKMaxTiles = 512;

// 16 x 16 int8 tiles for short panels: a workgroup of 8 waves owns one
// 16 x 16 output tile; each wave owns a run of up to 8 quads (4 blocks) of
// K (7 for 4-bit weights: at 8 the fused form would exceed the LDS).
// Measured on the decode-layer shapes at M = 8..64 (cold weights, one
// graph): 8 waves beat 4 and 16, and two or four row tiles per workgroup
// (weights read once) lost to one.
constexpr int64_t kTile16MaxQuads = 8;
constexpr int64_t kTile16MaxQuadsQ4 = 7;
struct Tile16Shape {
    int64_t waves, quads, mtiles;
};
constexpr Tile16Shape tile16_shape(int64_t /*M*/, int64_t /*N*/, int64_t K) {
    return {8, cdiv(cdiv(K / 32, 4), 8), 1};
}
constexpr int64_t tile16_quads_per_wave(int64_t K) { return tile16_shape(1, 1, K).quads; }

struct Q8Plan {
    Q8Kernel kernel;
    int64_t mt;     // Dot4: activation rows per pass; SplitK: 32-row tiles
    int64_t waves;  // SplitK: waves per workgroup
};

// Waves per split-K workgroup: a function of the format and the panel
// height only, so the fused 4-bit form adds its partial tiles in the same
// order as the plain product of the same shape.
constexpr int64_t splitk_waves(Fmt f, int64_t M) { return f == Fmt::Q8_0 && M <= 32 ? 16 : 8; }

// Short Q8_0 panels take the 16 x 16 tiles: one workgroup per output tile
// spreads the pp32 projections (28 to 152 tiles of 32 x 32) over the CUs.
// Measured against the dot4, staged-panel and split-K kernels (paired
// rounds, cold weights): the tiles win from 3 rows on (at 3 to 6 rows on the
// decode-layer shapes 3.6-4.2 against 5.0-6.0 us, the down projection 6.5-6.7
// against 7.2-8.1 us; 896 x 896 level), except for wide panels past 512
// tiles (M >= 32 over N = 4864), where split-K's 32 x 32 tiles read each
// weight once per 32 rows and are faster.  At 2 rows the staged panel keeps
// the fused 4-bit gate/up (30.8 against 35.2 us at 17408 x 5120).
constexpr int64_t kTile16MinRows = 3;
constexpr int64_t kTile16MaxRows = 64;
constexpr int64_t kTile16MaxTiles = 512;

// 4-bit weights take the tiles for one 16-row tile of activations (3 to 16
// rows, where the other choices are VALU dot4 kernels, the staged panel
// among them; the fused gate/up at 17408 x 5120 took 36 us on the
// persistent tiles at 3 to 8 rows against 38-54 us on the staged panel);
// from 17 rows on the 32 x 32 matrix-core kernels keep them.  The down projection of that
// FFN (K = 17408) has too many quads per wave and stays on the staged panel.
constexpr int64_t kTile16MaxRowsQ4 = 16;
constexpr bool tile16_preferred(Fmt f, int64_t M, int64_t N, int64_t K) {
    if (M < kTile16MinRows || tile16_quads_per_wave(K) > (f == Fmt::Q4 ? kTile16MaxQuadsQ4 : kTile16MaxQuads))
        return false;
    if (f == Fmt::Q4) return M <= kTile16MaxRowsQ4;
    return M <= kTile16MaxRows && (M <= 16 || cdiv(M, 16) * cdiv(N, 16) <= kTile16MaxTiles);
}

// M = 1: codes of 16 (Q8_0) or 32 (4-bit) per lane and sweep, loaded in
// groups of up to 8 sweeps per row (5 with two weight matrices, which at 8
// would not fit the 128 VGPRs of a 1024-thread workgroup).  The grouping
// does not change the order of the sums.  LDS holds the staged codes, one
// activation scale per chunk (and for 4-bit weights the chunk's code sum),
// for whole groups, and the outputs.
constexpr int64_t q8act_m1_max_group(int64_t nmat) { return nmat == 2 ? 5 : 8; }
constexpr int64_t q8act_m1_group(Fmt f, int64_t K, int64_t nmat) {
    const int64_t J = m1_sweeps(f, K);
    return cdiv(J, cdiv(J, q8act_m1_max_group(nmat)));
}
constexpr int64_t q8act_m1_lds_bytes(Fmt f, int64_t K, int64_t rows, int64_t nmat) {
    const int64_t S = q8act_m1_group(f, K, nmat);
    // per chunk: its codes, its scale and, for 4-bit weights, -8 x its code sum
    return cdiv(m1_sweeps(f, K), S) * S * kLanes * (chunk_codes(f) + 4 + (f == Fmt::Q4 ? 4 : 0)) + rows * 4;
}
// Waves per workgroup: the most of 16, 8 and 4 that spread the workgroup's
// rows within 10% of evenly (a wave takes every NW-th row, so the waves with
// one row more than the average set the time)
constexpr int64_t q8act_m1_waves(int64_t N, int64_t cus) {
    const int64_t rows = resident_rows(N, cus);
    for (int64_t nw = 16; nw >= 4; nw /= 2)
        if (10 * cdiv(rows, nw) * nw <= 11 * rows) return nw;
    return 4;
}
constexpr int64_t kQ8M1StageMinN = 4096;
constexpr bool q8act_m1_staged(Fmt f, int64_t M, int64_t N, int64_t K, int64_t cus) {
    return M == 1 && N >= kQ8M1StageMinN && q8act_m1_lds_bytes(f, K, resident_rows(N, cus), 2) <= kLdsBytes;
}

// The staged kernel can quantize an fp32 panel itself while staging it
// (quantize + product in one launch).  Its threads take the panel's groups
// of 8 values in rounds of one group each, loading up to kQ8M1QuantRounds
// rounds at once.  Measured against the two launches (quantize, then the
// staged product), on cold weights in paired graph rounds: one launch wins
// at K = 896 and 5120 (1-2 rounds; 4-bit gate/up 5120 -> 17408: 20.6
// against 21.9 us) and loses at K = 17408 over 256 threads (9 rounds; 4-bit
// down: 17.4 against 15.8 us), where every CU reads a 68 KB fp32 panel.
constexpr int64_t kQ8M1QuantRounds = 4;
constexpr bool q8act_m1_quantize_inside(Fmt f, int64_t M, int64_t N, int64_t K, int64_t cus) {
    return q8act_m1_staged(f, M, N, K, cus) && cdiv(K / 8, q8act_m1_waves(N, cus) * kLanes) <= kQ8M1QuantRounds;
}

// Panels of 2 .. 8 activation rows on the dot4 VALU path: one workgroup of
// 16 waves per CU stages the panel (M padded to MT = 2, 4 or 8 rows) in
// LDS, SW sweeps of 64 chunks per step in two buffers, and each wave takes
// RW weight rows (one register set of RW x SW chunks per matrix, two sets).
constexpr int64_t kPanelStagedMinN = 1024;
constexpr int64_t kPanelStagedMaxRows = 8;  // 16 rows of two matrices would not fit the registers
constexpr int64_t q8act_panel_mt(int64_t M) { return M <= 2 ? 2 : M <= 4 ? 4 : 8; }
// (two matrices take one sweep and one row per wave at a time, and 4-bit
// weights against 4 or more rows, or Q8_0 against 8, one sweep: with three
// register sets of weights more would not fit the 128 VGPRs of a
// 1024-thread workgroup)
constexpr int64_t q8act_panel_sweeps(Fmt f, int64_t mt, int64_t nmat) {
    return nmat == 2 || mt * (f == Fmt::Q4 ? 2 : 1) >= 8 ? 1 : 2;
}
constexpr int64_t q8act_panel_rows_per_wave(int64_t nmat) { return nmat == 2 ? 1 : 2; }
constexpr int64_t q8act_panel_lds_bytes(Fmt f, int64_t mt, int64_t nmat) {
    return 2 * mt * q8act_panel_sweeps(f, mt, nmat) * kLanes * (chunk_codes(f) + 4);
}
// rows per workgroup: the CU's share, at most 16 RW (one register row set per wave)
constexpr int64_t q8act_panel_rows(int64_t N, int64_t nmat, int64_t cus) {
    return imax(1, imin(16 * q8act_panel_rows_per_wave(nmat), cdiv(N, imax(1, cus))));
}
constexpr bool q8act_panel_staged(Fmt f, int64_t M, int64_t N, int64_t K) {
    (void)K;
    // the plain (larger) buffer decides, so the choice does not depend on the mode
    return M >= 2 && M <= kPanelStagedMaxRows && N >= kPanelStagedMinN &&
           q8act_panel_lds_bytes(f, q8act_panel_mt(M), 1) <= kLdsBytes;
}

// The persistent form of the 16 x 16 tiles: one workgroup of 8 waves per CU
// walks the weight tiles g, g + CUs, ...; wave w owns quads w Q .. w Q + Q - 1
// of K (activation operands kept in registers), loads its K slice of each
// tile's 16 rows as whole 16-byte chunks row after row, one tile ahead, and
// stages the tile through a private LDS region (rows one chunk apart, for
// conflict-free operand reads).  Measured on 17408 x 5120 at 8 to 16 rows
// (paired rounds): 4-bit plain 18.5 against 26.8 us for a tile per
// workgroup that read each instruction's 1 KB as 16 rows of 64 bytes, fused
// gate/up 36.9 against 43.1 us, Q8_0 at M = 16 25.0 against 46.8 us; against
// a tile per workgroup with the same loads it is level at one quad per wave
// (K <= 1024).  From 6 quads on (4-bit) or 7 (Q8_0) the fused or plain form
// would exceed the registers with two tiles' weights in them.
constexpr int64_t kPersistMinQuads = 2;
constexpr int64_t persist_max_quads(Fmt f) { return f == Fmt::Q4 ? 5 : 6; }
constexpr int64_t tile16_chunks_per_row(Fmt f, int64_t quads) { return quads * (f == Fmt::Q8_0 ? 8 : 4); }
constexpr int64_t tile16_stage_bytes(Fmt f, int64_t quads) {
    return 16 * (tile16_chunks_per_row(f, quads) + 1) * 16;
}
// one (two when persistent) buffer of 8 partial 16 x 16 tiles per matrix,
// then the waves' stages
constexpr int64_t tile16_lds_bytes(Fmt f, int64_t quads, int64_t nmat, bool persistent) {
    return (persistent ? 2 : 1) * nmat * 8 * 256 * 4 + 8 * nmat * tile16_stage_bytes(f, quads);
}
constexpr bool tile16_persistent(Fmt f, int64_t M, int64_t N, int64_t K, int64_t cus) {
    const int64_t quads = tile16_quads_per_wave(K);
    return M >= kTile16MinRows && M <= 16 && quads >= kPersistMinQuads && quads <= persist_max_quads(f) &&
           cdiv(N, 16) >= 2 * cus;
}

// The quantize-and-multiply calls at M = 1 on the per-row dot4 kernel: one
// launch whose every workgroup (4 rows) quantizes x itself, for rows of at
// most the sweeps its registers hold (8 for Q8_0, 4 for 4-bit), as long as
// the repeated quantization stays small (at most 2^21 elements over all
// workgroups; the 4864 x 896 gate and up quantize 1.1 M).  It takes these
// calls from the staged kernel too (the sums are the same, in the same
// order): at 4864 x 896 3.85 against 5.0 us.
constexpr int64_t kQ8M1QxMaxQuantized = int64_t{1} << 21;
constexpr bool q8act_m1_qx_per_row(Fmt f, int64_t M, int64_t N, int64_t K, int64_t /*cus*/) {
    return M == 1 && m1_sweeps(f, K) <= max_vgpr_sweeps(f) && cdiv(N, 4) * K <= kQ8M1QxMaxQuantized;
}

constexpr Q8Plan q8act_plan(Fmt f, int64_t M, int64_t N, int64_t K, int64_t cus) {
    if (q8act_m1_staged(f, M, N, K, cus)) return {Q8Kernel::M1Staged, 1, 16};
    if (tile16_persistent(f, M, N, K, cus)) return {Q8Kernel::Tile16Persist, 0, 8};
    if (tile16_preferred(f, M, N, K)) return {Q8Kernel::Tile16, 0, tile16_shape(M, N, K).waves};
    if (q8act_panel_staged(f, M, N, K)) return {Q8Kernel::PanelStaged, q8act_panel_mt(M), 16};
    if (M < kMfmaMinRows) return {Q8Kernel::Dot4, M == 1 ? 1 : (M == 2 ? 2 : 4), 0};
    if (M <= 64 && cdiv(M, 32) * cdiv(N, 32) < kSplitKMaxTiles)
        return {Q8Kernel::SplitK, M <= 32 ? 1 : 2, splitk_waves(f, M)};
    return {Q8Kernel::Panel, 0, 0};
}


}  // namespace plan
}  // namespace qbd
