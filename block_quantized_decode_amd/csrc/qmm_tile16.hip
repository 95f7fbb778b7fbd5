// Q8_0 or 4-bit weights x Q8 activations for short panels (8..64 activation
// rows) on 16 x 16 int8 matrix-core tiles: the pp32 prefill projections of
// Lumen v0.5.0 release page, "Headline" (32-token prompt) at every
// decode-layer shape, and the M = 8 4-bit FFN of LSE v0.4.16 release page,
// "Combined M8 Q4 gate/up execution", with the exact int32 block dot of
// Lumen v0.4.0 release page, "Phase 7.M - Q8xQ8 AVX2 int dot" and one fp32
// sub-accumulation per block ("Phase 7.O - 4-accumulator VNNI kernel", same
// page).
//
// qmm_q8_tile16: a workgroup of 8 waves owns the 16 weight rows of a tile
// column and 16 activation rows: one tile, so a 32-row panel over N weight
// rows gives 2 N / 16 workgroups (112 for N = 896, 608 for N = 4864), or, as
// the persistent form for one row group over at least two tiles per CU, one
// workgroup per CU that walks the tiles.  The waves split K by runs of quads
// of 4 blocks, and the 8 partial tiles are added in wave order through LDS;
// both forms form the same sums in the same order.
//
// Per quad (128 bytes of K of a Q8_0 row, 64 of a 4-bit row):
//   * Q8_0: each lane holds 16 bytes of one row twice (bytes 16 q and
//     64 + 16 q of the quad, lane l = 16 q + r for row r): one
//     v_permlane32_swap per dword pair turns them into the operands of four
//     v_mfma_i32_16x16x32_i8, one per block; the K order inside a block is a
//     fixed permutation, the same for weights and activations, so each MFMA
//     forms one whole block dot exactly in int32;
//   * 4-bit: lane 16 q + r holds block q of the quad for row r (16 bytes); a
//     4 x 4 transpose of dwords across the lane groups (four
//     v_permlane16/32_swap) leaves group g with dword g of every block, whose
//     low and high nibbles are codes 4g..4g+3 and 16+4g..16+4g+3: masked,
//     they are the operand as unsigned codes 0..15.  The activation operand
//     takes the same K slots (dwords g and 4 + g of the block, after two
//     transposes).  The -8 of each code enters through the MFMA's int32
//     input: one more MFMA against a constant -8 operand gives -8 times the
//     block's activation code sum, and the product starts from it, so the
//     block dot is again exact;
//   * one v_mfma_f32_16x16x1_4b_f32 forms the four blocks' scale outer
//     products d_x[m][b] * d_w[n][b] (one fp32 rounding each) in the result
//     layout of the dots: lanes 16 j .. 16 j + 15 supply block j;
//   * acc = fma(float(dot), scale, acc), blocks in order.
// The fused gate/up form (SwiGLU) keeps both matrices' tiles.  Rows past M or
// N and blocks past K are read from clamped, in-bounds addresses and meet a
// zero activation scale, so they add exactly zero.
#include "device_common.hpp"
#include "launch.hpp"

namespace qbd {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// v_permlane32_swap(a, b): a' = [a.lanes 0-31, b.lanes 0-31],
// b' = [a.lanes 32-63, b.lanes 32-63]
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
    auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// v_permlane16_swap(a, b): in 16-lane rows, a' = [a0 b0 a2 b2],
// b' = [a1 b1 a3 b3]
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
    auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// The two 16-byte loads of a lane (pieces p = 0, 1 of a quad: blocks 2p and
// 2p + 1) as four MFMA operands, one per block of the quad.  Before the
// swap, lanes 0-31 hold the first block of a piece, lanes 32-63 the second;
// after it, op[2p] holds the first block in every lane and op[2p + 1] the
// second.  K slots of a block: lanes 0-15 bytes 0-7, 16-31 bytes 16-23,
// 32-47 bytes 8-15, 48-63 bytes 24-31.
__device__ __forceinline__ void quad_operands(u4v lo, u4v hi, long (&op)[4]) {
    uint32_t a0 = lo[0], a1 = lo[1], a2 = lo[2], a3 = lo[3];
    uint32_t b0 = hi[0], b1 = hi[1], b2 = hi[2], b3 = hi[3];
    swap32(a0, a2);
    swap32(a1, a3);
    swap32(b0, b2);
    swap32(b1, b3);
    op[0] = static_cast<long>((static_cast<uint64_t>(a1) << 32) | a0);
    op[1] = static_cast<long>((static_cast<uint64_t>(a3) << 32) | a2);
    op[2] = static_cast<long>((static_cast<uint64_t>(b1) << 32) | b0);
    op[3] = static_cast<long>((static_cast<uint64_t>(b3) << 32) | b2);
}

// 4 x 4 transpose of dwords across the four 16-lane groups: register s of
// group g ends up with what register g of group s held.
__device__ __forceinline__ void transpose4(uint32_t& a, uint32_t& b, uint32_t& c, uint32_t& d) {
    swap32(a, c);
    swap32(b, d);
    swap16(a, b);
    swap16(c, d);
}

// 4-bit quads: K slots of lane group g in each block are codes 4g..4g+3
// (low nibbles of bytes 4g..4g+3) and 16+4g..16+4g+3 (the high nibbles of
// the same bytes).  Weights: group g loaded block g whole; after the
// transpose it holds dword g of every block, whose two nibble planes are the
// operand as unsigned codes 0..15 (the -8 goes in through the MFMA's C).
__device__ __forceinline__ void q4u_weight_operands(u4v w, long (&op)[4]) {
    uint32_t r[4] = {w[0], w[1], w[2], w[3]};
    transpose4(r[0], r[1], r[2], r[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = r[j] & 0x0F0F0F0Fu, hi = (r[j] >> 4) & 0x0F0F0F0Fu;
        op[j] = static_cast<long>((static_cast<uint64_t>(hi) << 32) | lo);
    }
}
// Activations for the same slots: group g loaded block g's 32 bytes as two
// 16-byte halves; after two transposes it holds dwords g and 4 + g of every
// block.
__device__ __forceinline__ void q4u_act_operands(u4v lo, u4v hi, long (&op)[4]) {
    uint32_t a[4] = {lo[0], lo[1], lo[2], lo[3]}, b[4] = {hi[0], hi[1], hi[2], hi[3]};
    transpose4(a[0], a[1], a[2], a[3]);
    transpose4(b[0], b[1], b[2], b[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) op[j] = static_cast<long>((static_cast<uint64_t>(b[j]) << 32) | a[j]);
}

// A workgroup of 8 waves takes the 16 x 16 output tiles of one row group
// mg (activation rows 16 mg .. 16 mg + 15): one tile (PERSIST false, one
// workgroup per tile), or the tiles g, g + G, ... of a grid of one workgroup
// per CU (PERSIST true, one row group).  Wave w always takes the Q
// consecutive quads w Q .. w Q + Q - 1 of K, so its activation operands are
// loaded and rearranged once and kept in registers.  Weight loads read whole
// 16-byte chunks of the wave's K slice, row after row (each instruction
// covers a few rows' full runs, not 16 rows' 64-byte pieces), into
// registers, one tile ahead when persistent; at its turn a tile goes through
// a private LDS region of the wave, from which each lane reads its MFMA
// operands.  The 8 partial tiles are added through LDS in wave order, so the
// two forms give the same bits.
template <Fmt F, int Q>
struct SliceShape {
    static constexpr int kQuadBytes = F == Fmt::Q8_0 ? 128 : 64;  // bytes of one quad in a weight row
    static constexpr int kCpr = static_cast<int>(plan::tile16_chunks_per_row(F, Q));  // 16-byte chunks per slice row
    static constexpr int kStride = kCpr + 1;                      // odd: conflict-free operand reads
    static constexpr int kLoads = 16 * kCpr / 64;                 // load instructions per matrix and tile
    static constexpr int kStageBytes = static_cast<int>(plan::tile16_stage_bytes(F, Q));  // one matrix, one wave
    static_assert(kStageBytes == 16 * kStride * 16 && kCpr % 4 == 0, "stage layout");
};

template <Fmt F, Mode MODE, int Q, bool PERSIST>
__global__ __launch_bounds__(512) void qmm_q8_tile16(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa, const uint8_t* __restrict__ wb,
    const uint16_t* __restrict__ sb, const int8_t* __restrict__ xq, const float* __restrict__ xd,
    float* __restrict__ y, int M, int N, int K, int n_tiles, int m_groups) {
    using S = SliceShape<F, Q>;
    constexpr int NW = 8;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    extern __shared__ __align__(16) uint8_t lds_t16[];
    float* red = reinterpret_cast<float*>(lds_t16);  // [2][NMAT][NW][256]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int NRED = PERSIST ? 2 : 1;
    u4v* stage = reinterpret_cast<u4v*>(lds_t16 + NRED * NMAT * NW * 256 * 4 + wave * NMAT * S::kStageBytes);
    const int r = lane & 15, q = lane >> 4;
    const int nb = K / kBlock;
    const int nquads = (nb + 3) / 4;
    const size_t rbytes = F == Fmt::Q8_0 ? static_cast<size_t>(K) : static_cast<size_t>(K) / 2;
    // items i = mg + m_groups nt; the grid is a multiple of m_groups, so a
    // persistent workgroup's tiles share one row group
    const int G = gridDim.x;
    int g = blockIdx.x;
    // one tile per workgroup and several row groups: XCD-contiguous ranges
    // (workgroup g runs on XCD g % 8), row groups fastest, so the row groups
    // of a weight tile share one L2
    if (!PERSIST && m_groups > 1 && (G & 7) == 0) g = (g & 7) * (G >> 3) + (g >> 3);
    const int mg = g % m_groups;
    const int Gt = G / m_groups;              // tile stride
    const int first = g / m_groups;           // first tile
    const int ntile_wg = first < n_tiles ? (n_tiles - 1 - first) / Gt + 1 : 0;
    const int row0 = 16 * mg;
    const int quad0 = wave * Q;  // first quad of this wave's K slice

    // ---- activation codes and scales of this wave's quads, loaded once
    u4v xraw[Q][2];
    float dx[Q];
    {
        const bool row_live = row0 + r < M;
        const int8_t* xrow = xq + static_cast<size_t>(min(row0 + r, M - 1)) * K;
        const float* xdrow = xd + static_cast<size_t>(min(row0 + r, M - 1)) * nb;
#pragma unroll
        for (int t = 0; t < Q; ++t) {
            const int quad_raw = quad0 + t;
            const int quad = min(quad_raw, nquads - 1);
            const int a0 = F == Fmt::Q8_0 ? 128 * quad + 16 * q : 128 * quad + 32 * q;
            const int a1 = F == Fmt::Q8_0 ? a0 + 64 : a0 + 16;
            xraw[t][0] = *reinterpret_cast<const u4v*>(xrow + min(a0, K - 16));
            xraw[t][1] = *reinterpret_cast<const u4v*>(xrow + min(a1, K - 16));
            const int b = 4 * quad_raw + q;
            // a multiply by 0 or 1, not a select: a select would put the
            // load under a branch of its own (the scale read is finite)
            const float live = quad_raw < nquads && b < nb && row_live ? 1.f : 0.f;
            dx[t] = xdrow[min(b, nb - 1)] * live;
        }
    }
    long xop[Q][4];

    // ---- one tile's weights for this wave's slice: chunk p = 64 i + lane
    // of load i is row p / kCpr, chunk p % kCpr of the slice
    struct Wt {
        u4v w[NMAT][S::kLoads];
        uint16_t s[NMAT][Q];
    };
    const size_t slice0 = static_cast<size_t>(quad0) * S::kQuadBytes;
    auto wload = [&](Wt& T, int k) {
        const int nt = first + Gt * k;
#pragma unroll
        for (int i = 0; i < S::kLoads; ++i) {
            const int p = 64 * i + lane;
            const int n = min(nt * 16 + p / S::kCpr, N - 1);
            const size_t off = min(slice0 + 16 * static_cast<size_t>(p % S::kCpr), rbytes - 16);
#pragma unroll
            for (int q2 = 0; q2 < NMAT; ++q2) {
                const u4v* src = reinterpret_cast<const u4v*>((q2 == 0 ? wa : wb) + static_cast<size_t>(n) * rbytes + off);
                // persistent: plain loads, so the half line that two waves'
                // slices share stays in L2 for the second one (non-temporal
                // loads fetched 21% over the weight bytes and ran 4-7%
                // slower); one tile per workgroup: non-temporal (measured
                // level or faster)
                if constexpr (PERSIST)
                    T.w[q2][i] = *src;
                else
                    T.w[q2][i] = __builtin_nontemporal_load(src);
            }
        }
        const int n = min(nt * 16 + r, N - 1);
#pragma unroll
        for (int t = 0; t < Q; ++t) {
            const int b = min(4 * (quad0 + t) + q, nb - 1);
#pragma unroll
            for (int q2 = 0; q2 < NMAT; ++q2) T.s[q2][t] = (q2 == 0 ? sa : sb)[static_cast<size_t>(n) * nb + b];
        }
    };

    const v4i zi = {0, 0, 0, 0};
    const v16f zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto tile = [&](const Wt& T, int k) {
        // the tile's slice into this wave's LDS region, rows kStride chunks apart
#pragma unroll
        for (int i = 0; i < S::kLoads; ++i) {
            const int p = 64 * i + lane;
            const int at = (p / S::kCpr) * S::kStride + p % S::kCpr;
#pragma unroll
            for (int q2 = 0; q2 < NMAT; ++q2) stage[q2 * (S::kStageBytes / 16) + at] = T.w[q2][i];
        }
        v4f acc[NMAT];
#pragma unroll
        for (int q2 = 0; q2 < NMAT; ++q2) acc[q2] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < Q; ++t) {
            long wop[NMAT][4];
            float dw[NMAT];
#pragma unroll
            for (int q2 = 0; q2 < NMAT; ++q2) {
                const u4v* sr = stage + q2 * (S::kStageBytes / 16) + r * S::kStride;
                if constexpr (F == Fmt::Q8_0)
                    quad_operands(sr[8 * t + q], sr[8 * t + 4 + q], wop[q2]);
                else
                    q4u_weight_operands(sr[4 * t + q], wop[q2]);
                dw[q2] = f16_bits_to_f32(T.s[q2][t]);
            }
            v4i base[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (F == Fmt::Q8_0) {
                    base[j] = zi;
                } else {
                    constexpr long kMinus8 = static_cast<long>(0xF8F8F8F8F8F8F8F8ull);
                    base[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(xop[t][j], kMinus8, zi, 0, 0, 0);
                }
            }
            v16f sc[NMAT];
#pragma unroll
            for (int q2 = 0; q2 < NMAT; ++q2) sc[q2] = __builtin_amdgcn_mfma_f32_16x16x1f32(dx[t], dw[q2], zf, 0, 0, 0);
            // block j's products are issued before block j - 1's are
            // consumed, so each MFMA's latency is covered by VALU work
            v4i dot[2][NMAT];
#pragma unroll
            for (int q2 = 0; q2 < NMAT; ++q2)
                dot[0][q2] = __builtin_amdgcn_mfma_i32_16x16x32_i8(xop[t][0], wop[q2][0], base[0], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j + 1 < 4) {
#pragma unroll
                    for (int q2 = 0; q2 < NMAT; ++q2)
                        dot[(j + 1) & 1][q2] =
                            __builtin_amdgcn_mfma_i32_16x16x32_i8(xop[t][j + 1], wop[q2][j + 1], base[j + 1], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q2 = 0; q2 < NMAT; ++q2)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[q2][e] = __builtin_fmaf(static_cast<float>(dot[j & 1][q2][e]), sc[q2][4 * j + e], acc[q2][e]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // partial tiles through LDS, added in wave order
        float* buf = red + (PERSIST ? (k & 1) : 0) * NMAT * NW * 256;
#pragma unroll
        for (int q2 = 0; q2 < NMAT; ++q2)
#pragma unroll
            for (int e = 0; e < 4; ++e) buf[(q2 * NW + wave) * 256 + e * 64 + lane] = acc[q2][e];
        __syncthreads();
        if (threadIdx.x < 256) {
            const int el = threadIdx.x;
            float v[NMAT];
#pragma unroll
            for (int q2 = 0; q2 < NMAT; ++q2) {
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sum += buf[(q2 * NW + w) * 256 + el];
                v[q2] = sum;
            }
            const int e = el >> 6, l = el & 63;
            const int row = row0 + 4 * (l >> 4) + e, col = (first + Gt * k) * 16 + (l & 15);
            if (row < M && col < N)
                y[static_cast<size_t>(row) * N + col] = MODE == Mode::SwiGLU ? swiglu_f32(v[0], v[NMAT - 1]) : v[0];
        }
    };

    if (ntile_wg == 0) return;  // workgroup-uniform
    const int last = ntile_wg - 1;
    Wt A, B;
    wload(A, 0);  // in flight while the activation operands are formed
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < Q; ++t) {
        if constexpr (F == Fmt::Q8_0)
            quad_operands(xraw[t][0], xraw[t][1], xop[t]);
        else
            q4u_act_operands(xraw[t][0], xraw[t][1], xop[t]);
    }
    if constexpr (!PERSIST) {
        tile(A, 0);
        return;
    }
    for (int k = 0; k < ntile_wg; k += 2) {
        wload(B, min(k + 1, last));
        __builtin_amdgcn_sched_barrier(0);
        tile(A, k);
        if (k + 1 >= ntile_wg) break;
        wload(A, min(k + 2, last));
        __builtin_amdgcn_sched_barrier(0);
        tile(B, k + 1);
    }
}

template <Fmt F, Mode MODE, int Q, bool PERSIST>
hipError_t launch_tile_q(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb, const int8_t* xq,
                         const float* xd, float* y, int M, int N, int K, int G, int m_groups, hipStream_t stream) {
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr size_t lds = static_cast<size_t>(plan::tile16_lds_bytes(F, Q, NMAT, PERSIST));
    static_assert(lds <= static_cast<size_t>(plan::kLdsBytes), "16 x 16 tile LDS");
    static_assert(lds == static_cast<size_t>((PERSIST ? 2 : 1) * NMAT * 8 * 256 * 4 + 8 * NMAT * SliceShape<F, Q>::kStageBytes),
                  "LDS layout");
    hipLaunchKernelGGL((qmm_q8_tile16<F, MODE, Q, PERSIST>), dim3(G), dim3(512), lds, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb, xq, xd, y, M, N, K,
                       (N + 15) / 16, m_groups);
    return hipGetLastError();
}

// quads per wave: 1..8 for one tile per workgroup (4-bit: up to 7), 2..6
// persistent (4-bit: up to 5); the plan keeps to these
template <Fmt F, Mode MODE, bool PERSIST>
hipError_t launch_tile(int quads, const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                       const int8_t* xq, const float* xd, float* y, int M, int N, int K, int G, int m_groups,
                       hipStream_t stream) {
    constexpr int kMax = PERSIST ? static_cast<int>(plan::persist_max_quads(F))
                                 : static_cast<int>(F == Fmt::Q4 ? plan::kTile16MaxQuadsQ4 : plan::kTile16MaxQuads);
    if (quads < 1 || quads > kMax) return hipErrorInvalidValue;
    switch (quads) {
        case 1: return launch_tile_q<F, MODE, 1, PERSIST>(wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups, stream);
        case 2: return launch_tile_q<F, MODE, 2, PERSIST>(wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups, stream);
        case 3: return launch_tile_q<F, MODE, 3, PERSIST>(wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups, stream);
        case 4: return launch_tile_q<F, MODE, 4, PERSIST>(wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups, stream);
        case 5: return launch_tile_q<F, MODE, 5, PERSIST>(wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups, stream);
        case 6:
            if constexpr (kMax >= 6)
                return launch_tile_q<F, MODE, 6, PERSIST>(wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups, stream);
            return hipErrorInvalidValue;
        case 7:
            if constexpr (kMax >= 7)
                return launch_tile_q<F, MODE, 7, PERSIST>(wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups, stream);
            return hipErrorInvalidValue;
        case 8:
            if constexpr (kMax >= 8)
                return launch_tile_q<F, MODE, 8, PERSIST>(wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups, stream);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <bool PERSIST>
hipError_t launch_tile_any(Fmt fmt, Mode mode, int quads, const void* wa, const uint16_t* sa, const void* wb,
                           const uint16_t* sb, const int8_t* xq, const float* xd, float* y, int M, int N, int K,
                           int G, int m_groups, hipStream_t stream) {
    if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
        return launch_tile<Fmt::Q8_0, Mode::Plain, PERSIST>(quads, wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups,
                                                            stream);
    if (fmt == Fmt::Q4 && mode == Mode::Plain)
        return launch_tile<Fmt::Q4, Mode::Plain, PERSIST>(quads, wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups,
                                                          stream);
    if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
        return launch_tile<Fmt::Q4, Mode::SwiGLU, PERSIST>(quads, wa, sa, wb, sb, xq, xd, y, M, N, K, G, m_groups,
                                                           stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qmm_q8_tile16(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa, const void* wb,
                                const uint16_t* sb, const int8_t* xq, const float* xd, float* y, int64_t M,
                                int64_t N, int64_t K, hipStream_t stream) {
    if (!plan::tile16_preferred(fmt, M, N, K)) return hipErrorInvalidValue;
    const int64_t m_groups = plan::cdiv(M, 16), tiles = m_groups * plan::cdiv(N, 16);
    if (tiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    return launch_tile_any<false>(fmt, mode, static_cast<int>(plan::tile16_quads_per_wave(K)), wa, sa, wb, sb, xq,
                                  xd, y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K),
                                  static_cast<int>(tiles), static_cast<int>(m_groups), stream);
}

hipError_t launch_qmm_q8_tile16_persist(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa, const void* wb,
                                        const uint16_t* sb, const int8_t* xq, const float* xd, float* y, int64_t M,
                                        int64_t N, int64_t K, hipStream_t stream) {
    const int cus = device_cus();
    if (!plan::tile16_persistent(fmt, M, N, K, cus)) return hipErrorInvalidValue;
    // one workgroup per CU; every one of them has at least two tiles
    return launch_tile_any<true>(fmt, mode, static_cast<int>(plan::tile16_quads_per_wave(K)), wa, sa, wb, sb, xq,
                                 xd, y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), cus, 1,
                                 stream);
}

}  // namespace qbd
