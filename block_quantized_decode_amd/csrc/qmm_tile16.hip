// Q8_0 weights x Q8 activations for short panels (2..64 activation rows) on
// 16 x 16 int8 matrix-core tiles: the pp32 prefill projections of Lumen
// v0.5.0 release page, "Headline" (32-token prompt) at every decode-layer
// shape, with the exact int32 block dot of Lumen v0.4.0 release page,
// "Phase 7.M - Q8xQ8 AVX2 int dot" and one fp32 sub-accumulation per block
// ("Phase 7.O - 4-accumulator VNNI kernel", same page).
//
// A workgroup owns the 16 weight rows of one tile column and MT tiles of 16
// activation rows, so a 32-row panel over N weight rows gives up to 2 N / 16
// workgroups: 112 for N = 896, 608 for N = 4864, enough to spread the short
// launches over the 256 CUs.  Its NW waves split K by quads of 4 blocks
// (quad t of wave w: t = w, w + NW, ...), and each wave issues the loads of
// all its quads before any arithmetic, so one memory round trip covers the
// whole K range.  The NW partial tiles are added in wave order through LDS.
//
// Per quad (128 bytes of K):
//   * each lane loads 16 bytes of one row twice (bytes 16 q and 64 + 16 q
//     of the quad, lane l = 16 q + r reading row r): one v_permlane32_swap
//     per dword pair turns the two loads into the operands of four
//     v_mfma_i32_16x16x32_i8, one per block; the K order inside a block is
//     a fixed permutation, the same for weights and activations, so each
//     MFMA forms one whole block dot exactly in int32;
//   * one v_mfma_f32_16x16x1_4b_f32 forms the four blocks' scale outer
//     products d_x[m][b] * d_w[n][b] (one fp32 rounding each) in the result
//     layout of the dots: lanes 16 j .. 16 j + 15 supply block j;
//   * acc = fma(float(dot), scale, acc), blocks in order.
// 4-bit weights (Q4; the prefill panels of LSE v0.4.16 release page,
// "Retained optimizations and compatibility", at short panels) load one
// 16-byte block per lane and quad (lane 16 q + r: block q of the quad, row
// r); a 4 x 4 transpose of dwords across the lane groups (four
// v_permlane16/32_swap) leaves lane group g with dword g of each block, and
// one more swap per block shares each 8-byte half between the two groups
// that need it: groups 0 and 1 take the low and the high nibbles of bytes
// 0-7 (codes 0-7 and 16-23), groups 2 and 3 those of bytes 8-15 (codes 8-15
// and 24-31), the K slots of the activation operands.  Each nibble becomes
// the signed byte q - 8, so the MFMA forms the block dot exactly, as for
// Q8_0.  The fused gate/up form (SwiGLU) keeps both matrices' tiles.
// Rows past M or N and blocks past K are read from clamped, in-bounds
// addresses and meet a zero activation scale, so they add exactly zero.
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

// 4 nibbles (low or high halves, by the shift) as signed bytes q - 8
__device__ __forceinline__ uint32_t q4_s8(uint32_t w, int shift) {
    return (((w >> shift) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
}

// The four MFMA operands of a 4-bit quad from one 16-byte load per lane
// (lane group g = lane / 16 loaded block g whole).
__device__ __forceinline__ void q4_quad_operands(u4v w, int lane, long (&op)[4]) {
    uint32_t a = w[0], b = w[1], c = w[2], d = w[3];
    // transpose: register s then holds dword g of block s
    swap32(a, c);
    swap32(b, d);
    swap16(a, b);
    swap16(c, d);
    const uint32_t blk[4] = {a, b, c, d};
    const int shift = (lane >> 4) & 1 ? 4 : 0;  // groups 1, 3: high nibbles
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // groups 0, 1 get dwords 0, 1 of block j; groups 2, 3 dwords 2, 3
        uint32_t lo = blk[j], hi = blk[j];
        swap16(lo, hi);
        op[j] = static_cast<long>((static_cast<uint64_t>(q4_s8(hi, shift)) << 32) | q4_s8(lo, shift));
    }
}

template <Fmt F, Mode MODE, int NW, int Q, int MT>
__global__ __launch_bounds__(NW * 64) void qmm_q8_tile16(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa, const uint8_t* __restrict__ wb,
    const uint16_t* __restrict__ sb, const int8_t* __restrict__ xq, const float* __restrict__ xd,
    float* __restrict__ y, int M, int N, int K, int m_groups, int n_tiles) {
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    __shared__ float red[NW * MT * NMAT * 256];
    const int total = m_groups * n_tiles;
    int g = blockIdx.x;
    // XCD-contiguous tile ranges (workgroup g runs on XCD g % 8), M fastest:
    // the row tiles that share a weight tile share one L2
    if ((total & 7) == 0) g = (g & 7) * (total >> 3) + (g >> 3);
    const int mg = g % m_groups, nt = g / m_groups;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int nb = K / kBlock;
    const int nquads = (nb + 3) / 4;
    const int n = nt * 16 + r;
    const size_t rbytes = F == Fmt::Q8_0 ? static_cast<size_t>(K) : static_cast<size_t>(K) / 2;
    const uint8_t* wrow[NMAT];
    const uint16_t* wdrow[NMAT];
#pragma unroll
    for (int q2 = 0; q2 < NMAT; ++q2) {
        wrow[q2] = (q2 == 0 ? wa : wb) + static_cast<size_t>(min(n, N - 1)) * rbytes;
        wdrow[q2] = (q2 == 0 ? sa : sb) + static_cast<size_t>(min(n, N - 1)) * nb;
    }
    const int8_t* xrow[MT];
    const float* xdrow[MT];
    bool row_live[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = (mg * MT + i) * 16 + r;
        row_live[i] = m < M;
        xrow[i] = xq + static_cast<size_t>(min(m, M - 1)) * K;
        xdrow[i] = xd + static_cast<size_t>(min(m, M - 1)) * nb;
    }

    // ---- every load of this wave's quads, before any arithmetic
    constexpr int WL = F == Fmt::Q8_0 ? 2 : 1;  // 16-byte weight loads per lane and quad
    u4v wv[NMAT][Q][WL], xl[Q][MT], xh[Q][MT];
    float dxs[Q][MT];
    uint16_t dws[NMAT][Q];
#pragma unroll
    for (int t = 0; t < Q; ++t) {
        const int quad = min(wave + NW * t, nquads - 1);
        const int off0 = min(128 * quad + 16 * q, K - 16);
        const int off1 = min(128 * quad + 64 + 16 * q, K - 16);
        const int b = min(4 * quad + q, nb - 1);
#pragma unroll
        for (int q2 = 0; q2 < NMAT; ++q2) {
            if constexpr (F == Fmt::Q8_0) {
                wv[q2][t][0] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(wrow[q2] + off0));
                wv[q2][t][WL - 1] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(wrow[q2] + off1));
            } else {
                // block b whole (16 bytes of nibbles)
                wv[q2][t][0] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(wrow[q2] + 16 * static_cast<size_t>(b)));
            }
            dws[q2][t] = wdrow[q2][b];
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            xl[t][i] = *reinterpret_cast<const u4v*>(xrow[i] + off0);
            xh[t][i] = *reinterpret_cast<const u4v*>(xrow[i] + off1);
            dxs[t][i] = xdrow[i][b];
        }
    }


    v4f acc[NMAT][MT];
#pragma unroll
    for (int q2 = 0; q2 < NMAT; ++q2)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[q2][i] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4i zi = {0, 0, 0, 0};
    const v16f zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < Q; ++t) {
        // (the compiler moves each quad's loads down to this test; keeping
        // every load above the arithmetic instead, by multiplying the slots
        // past the last quad with a zero scale, raised the registers to up to
        // 192 and ran slower: fewer workgroups per CU overlapped less memory)
        const int quad = wave + NW * t;
        if (quad >= nquads) break;  // wave-uniform
        long wop[NMAT][4];
        float dw[NMAT];
#pragma unroll
        for (int q2 = 0; q2 < NMAT; ++q2) {
            if constexpr (F == Fmt::Q8_0) {
                quad_operands(wv[q2][t][0], wv[q2][t][WL - 1], wop[q2]);
            } else {
                q4_quad_operands(wv[q2][t][0], lane, wop[q2]);
            }
            dw[q2] = f16_bits_to_f32(dws[q2][t]);
        }
        const bool block_live = 4 * quad + q < nb;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            long xop[4];
            quad_operands(xl[t][i], xh[t][i], xop);
            // blocks past K and rows past M meet a zero activation scale
            const float dx = block_live && row_live[i] ? dxs[t][i] : 0.f;
#pragma unroll
            for (int q2 = 0; q2 < NMAT; ++q2) {
                const v16f sc = __builtin_amdgcn_mfma_f32_16x16x1f32(dx, dw[q2], zf, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4i dot = __builtin_amdgcn_mfma_i32_16x16x32_i8(xop[j], wop[q2][j], zi, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[q2][i][e] = __builtin_fmaf(static_cast<float>(dot[e]), sc[4 * j + e], acc[q2][i][e]);
                }
            }
        }
    }

    // ---- partial tiles added in wave order; D layout: lane l, register e ->
    // activation row 4 (l / 16) + e, weight row l % 16
#pragma unroll
    for (int q2 = 0; q2 < NMAT; ++q2)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[((q2 * NW + wave) * MT + i) * 256 + e * 64 + lane] = acc[q2][i][e];
    __syncthreads();
    for (int t = threadIdx.x; t < MT * 256; t += NW * 64) {
        const int i = t >> 8, el = t & 255;
        float v[NMAT];
#pragma unroll
        for (int q2 = 0; q2 < NMAT; ++q2) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) s += red[((q2 * NW + w) * MT + i) * 256 + el];
            v[q2] = s;
        }
        const int e = el >> 6, l = el & 63;
        const int row = (mg * MT + i) * 16 + 4 * (l >> 4) + e, col = nt * 16 + (l & 15);
        if (row < M && col < N)
            y[static_cast<size_t>(row) * N + col] = MODE == Mode::SwiGLU ? swiglu_f32(v[0], v[NMAT - 1]) : v[0];
    }
}

template <Fmt F, Mode MODE, int NW, int Q, int MT>
hipError_t launch_q(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb, const int8_t* xq,
                    const float* xd, float* y, int M, int N, int K, hipStream_t stream) {
    const int m_groups = (M + 16 * MT - 1) / (16 * MT), n_tiles = (N + 15) / 16;
    const long long total = static_cast<long long>(m_groups) * n_tiles;
    if (total > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((qmm_q8_tile16<F, MODE, NW, Q, MT>), dim3(static_cast<unsigned>(total)), dim3(NW * 64), 0,
                       stream, static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb, xq, xd, y, M,
                       N, K, m_groups, n_tiles);
    return hipGetLastError();
}

template <Fmt F, Mode MODE, int NW, int MT>
hipError_t launch_nw(int quads, const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                     const int8_t* xq, const float* xd, float* y, int M, int N, int K, hipStream_t stream) {
    switch (quads) {
        case 1: return launch_q<F, MODE, NW, 1, MT>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 2: return launch_q<F, MODE, NW, 2, MT>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 3: return launch_q<F, MODE, NW, 3, MT>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 4: return launch_q<F, MODE, NW, 4, MT>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 5: return launch_q<F, MODE, NW, 5, MT>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 6: return launch_q<F, MODE, NW, 6, MT>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 7: return launch_q<F, MODE, NW, 7, MT>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 8: return launch_q<F, MODE, NW, 8, MT>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_qmm_q8_tile16(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa, const void* wb,
                                const uint16_t* sb, const int8_t* xq, const float* xd, float* y, int64_t M,
                                int64_t N, int64_t K, hipStream_t stream) {
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    const plan::Tile16Shape t = plan::tile16_shape(M, N, K);
    if (t.waves != 8 || t.mtiles != 1) return hipErrorInvalidValue;
    const int quads = static_cast<int>(t.quads);
    if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
        return launch_nw<Fmt::Q8_0, Mode::Plain, 8, 1>(quads, wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
    if (fmt == Fmt::Q4 && mode == Mode::Plain)
        return launch_nw<Fmt::Q4, Mode::Plain, 8, 1>(quads, wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
    if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
        return launch_nw<Fmt::Q4, Mode::SwiGLU, 8, 1>(quads, wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
    return hipErrorInvalidValue;
}

}  // namespace qbd
