// Weights x Q8 activations on the gfx950 matrix cores, for panels of 32 or
// more activation rows (the pp32 prefill of Lumen v0.5.0 release page,
// "Headline"; the M1024 prefill panels of LSE v0.4.16 release page,
// "Retained optimizations and compatibility").
//
// y[m,n] = sum_b (d_w[n,b] * d_x[m,b]) * dot[m,n,b]:
//   * dot: one v_mfma_i32_32x32x32_i8 per 32 x 32 output tile and block -
//     its K of 32 is exactly one quantization block, so every block dot is
//     formed whole and exactly in int32 (Lumen v0.4.0 release page, "Phase
//     7.M - Q8xQ8 AVX2 int dot");
//   * d_x[m,b] * d_w[n,b] for the same tile: the rank-1 outer product,
//     produced in the same lane layout as the dots (each product is one fp32
//     rounding) - in the main kernels one v_mfma_f32_32x32x1_2b_f32 for two
//     consecutive blocks at once (lane half h gives block 2i + h), in the
//     short-panel split-K kernel one v_mfma_f32_32x32x2_f32 with a single
//     nonzero k;
//   * acc = fma(float(dot), scale, acc) on the VALU, blocks in order, one
//     fp32 sub-accumulation per block ("Phase 7.O - 4-accumulator VNNI
//     kernel", same page).
// 4-bit weights become the int8 codes 16 (q - 8) byte-parallel (bit 3 of
// each nibble flipped, the nibble moved to the top of its byte), with the
// weight scale taken as d / 16.
//
// Tiling: a workgroup of 4 waves (WGM along M x WGN along N), each wave
// owning TM x TN tiles of 32 x 32 per weight matrix (two matrices in the
// SwiGLU mode).  K is walked in stages of a few blocks: the workgroup
// loads a stage of its activation rows and weight columns (whole 16-byte
// row pieces, coalesced) into LDS, and the waves read their fragments
// there while the next stage is in flight.  Two kernels do this: one that
// copies the stage straight into LDS (global_load_lds, for K in whole
// 4-block stages and aligned rows) and one that stages it through
// registers (any K).  Workgroups are numbered so that the tiles sharing one
// weight panel run on one XCD (one L2).  Short panels with few output
// tiles take a split-K kernel instead (below).
#include "device_common.hpp"
#include "launch.hpp"

namespace qbd {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
// native vector for staging registers (HIP's uint4 class can defeat the
// promotion of register arrays and land them in scratch)
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

// 4-bit codes of one nibble half as signed bytes 16 (q - 8): bit 3 of each
// nibble flipped makes it the two's-complement q - 8, and the nibble moved
// to the top of its byte reads 16 (q - 8).  `up` = 4 takes the low nibbles
// (shifted up), 0 the high ones.  The block dot is then 16x the dot of the
// codes q - 8 (|16 dot| < 2^20, exact in int32 and in fp32), and the weight
// scale is taken as d / 16 (Frag::scale), so float(dot) * scale is exactly
// the product of the plain dot and d.
__device__ __forceinline__ uint32_t q4x16_half(uint32_t w, int up) {
    return ((w << up) & 0xF0F0F0F0u) ^ 0x80808080u;
}

template <Fmt F>
struct Frag {
    // B fragment of 32 x 32 x 32: lane (j = l % 32, h = l / 32) holds the
    // 16 codes k = 16h .. 16h + 15 of column j of block b.
    static __device__ __forceinline__ const uint8_t* col_ptr(const uint8_t* w, int col, int K, int h) {
        if constexpr (F == Fmt::Q8_0) return w + static_cast<size_t>(col) * K + 16 * h;
        else return w + static_cast<size_t>(col) * (K / 2);
    }
    static __device__ __forceinline__ uint4 load(const uint8_t* p, int b) {
        if constexpr (F == Fmt::Q8_0) return *reinterpret_cast<const uint4*>(p + 32 * b);
        else return *reinterpret_cast<const uint4*>(p + 16 * b);
    }
    static __device__ __forceinline__ v4i codes(uint4 raw, int h) {
        v4i r;
        if constexpr (F == Fmt::Q8_0) {
            r[0] = static_cast<int>(raw.x); r[1] = static_cast<int>(raw.y);
            r[2] = static_cast<int>(raw.z); r[3] = static_cast<int>(raw.w);
        } else {
            const int up = 4 - 4 * h;  // low nibbles: codes 0..15, high: 16..31
            r[0] = static_cast<int>(q4x16_half(raw.x, up)); r[1] = static_cast<int>(q4x16_half(raw.y, up));
            r[2] = static_cast<int>(q4x16_half(raw.z, up)); r[3] = static_cast<int>(q4x16_half(raw.w, up));
        }
        return r;
    }
    // weight scale paired with codes(): d, or d / 16 for 4-bit codes (exact)
    static __device__ __forceinline__ float scale(uint16_t bits) {
        return F == Fmt::Q8_0 ? f16_bits_to_f32(bits) : f16_bits_to_f32(bits) * 0.0625f;
    }
};

// Register-staged kernel.  A stage holds KS blocks of K for the
// workgroup's BM activation rows and BN weight columns (per matrix), plus
// their scales; rows are padded by 16 bytes so that the per-lane 16-byte
// fragment reads of 8 consecutive rows fall in distinct banks.
template <Fmt F, Mode MODE, int WGM, int WGN, int TM, int TN, int KS>
struct Tile {
    static constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    static constexpr int BM = 32 * TM * WGM;            // activation rows
    static constexpr int BN = 32 * TN * WGN;            // weight columns per matrix
    static constexpr int WBYTES = F == Fmt::Q8_0 ? 32 : 16;  // weight bytes per block
    static constexpr int A_STRIDE = 32 * KS + 16;
    static constexpr int B_STRIDE = WBYTES * KS + 16;
    static constexpr int A_BYTES = BM * A_STRIDE;
    static constexpr int B_BYTES = NMAT * BN * B_STRIDE;
    static constexpr int DX_BYTES = BM * KS * 4;
    static constexpr int DW_BYTES = NMAT * BN * KS * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES + DX_BYTES + DW_BYTES;
    // 16-byte chunks (and scale words) per stage, and per thread
    static constexpr int A_TOTAL = BM * 2 * KS;                 // 32*KS bytes per row
    static constexpr int B_TOTAL = NMAT * BN * (WBYTES * KS / 16);
    static constexpr int A_CHUNKS = (A_TOTAL + 255) / 256;
    static constexpr int B_CHUNKS = (B_TOTAL + 255) / 256;
    static constexpr int DX_ITEMS = (BM * KS + 255) / 256;
    static constexpr int DW_ITEMS = (NMAT * BN * KS + 255) / 256;
};

// Register budget: two waves per SIMD (256 VGPRs).  The staging registers
// of a whole stage do not fit the 168 VGPRs of three waves without spilling.
template <Fmt F, Mode MODE, int WGM, int WGN, int TM, int TN, int KS>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(2)))
void qmm_mfma_kernel(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, float* __restrict__ y,
    int M, int N, int K, int m_tiles, int n_tiles) {
    static_assert(WGM * WGN == 4, "four waves per workgroup");
    using T = Tile<F, MODE, WGM, WGN, TM, TN, KS>;
    constexpr int NMAT = T::NMAT;
    extern __shared__ __align__(16) uint8_t lds[];

    // XCD-aware order: workgroup g runs on XCD g % 8; give each XCD a
    // contiguous range of the M-fastest tile order, so the M tiles that
    // share a weight panel stay in one L2.
    const int total = m_tiles * n_tiles;
    int g = blockIdx.x;
    if ((total & 7) == 0) g = (g & 7) * (total >> 3) + (g >> 3);
    const int mt = g % m_tiles, nt = g / m_tiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int wm = wave % WGM, wn = wave / WGM;
    const int mbase = mt * T::BM, nbase = nt * T::BN;
    const int nb = K / kBlock;
    const int stages = (nb + KS - 1) / KS;
    const size_t wrow = F == Fmt::Q8_0 ? static_cast<size_t>(K) : static_cast<size_t>(K) / 2;

    // ---- global -> registers -> LDS staging of one stage
    u4v ra[T::A_CHUNKS], rb[T::B_CHUNKS];
    float rdx[T::DX_ITEMS];
    uint16_t rdw[T::DW_ITEMS];
    auto gload = [&](int st) {
        const int b0 = st * KS;
#pragma unroll
        for (int u = 0; u < T::A_CHUNKS; ++u) {
            const int c = min(tid + 256 * u, T::A_TOTAL - 1);        // extra threads repeat the last chunk
            const int row = c / (2 * KS), part = c % (2 * KS);       // 16-byte part of the row
            const int r = min(mbase + row, M - 1);
            const int blk = min(b0 + part / 2, nb - 1);
            ra[u] = *reinterpret_cast<const u4v*>(xq + static_cast<size_t>(r) * K + 32 * blk + 16 * (part & 1));
        }
        constexpr int BPARTS = T::WBYTES * KS / 16;  // 16-byte parts per column per stage
        constexpr int BPB = T::WBYTES / 16;          // parts per block
#pragma unroll
        for (int u = 0; u < T::B_CHUNKS; ++u) {
            const int c = min(tid + 256 * u, T::B_TOTAL - 1);
            const int colx = c / BPARTS, part = c % BPARTS;
            const int q = colx / T::BN, col = colx % T::BN;
            const int cc = min(nbase + col, N - 1);
            const int blk = min(b0 + part / BPB, nb - 1);
            const uint8_t* w = (NMAT == 2 && q == 1) ? wb : wa;
            rb[u] = *reinterpret_cast<const u4v*>(w + static_cast<size_t>(cc) * wrow + T::WBYTES * blk + 16 * (part % BPB));
        }
        // scale words: every thread loads (clamped, in bounds) so that no
        // load sits under a branch that would wait for it at once; the zero
        // of blocks past K and the fp16 decode happen at the LDS store
#pragma unroll
        for (int u = 0; u < T::DX_ITEMS; ++u) {
            const int c = min(tid + 256 * u, T::BM * KS - 1);
            const int row = c / KS, kb = c % KS;
            const int r = min(mbase + row, M - 1);
            const int blk = min(b0 + kb, nb - 1);
            rdx[u] = xd[static_cast<size_t>(r) * nb + blk];
        }
#pragma unroll
        for (int u = 0; u < T::DW_ITEMS; ++u) {
            const int c = min(tid + 256 * u, NMAT * T::BN * KS - 1);
            const int colx = c / KS, kb = c % KS;
            const int q = colx / T::BN, col = colx % T::BN;
            const int cc = min(nbase + col, N - 1);
            const int blk = min(b0 + kb, nb - 1);
            const uint16_t* s = (NMAT == 2 && q == 1) ? sb : sa;
            rdw[u] = s[static_cast<size_t>(cc) * nb + blk];
        }
    };
    auto lstore = [&](uint8_t* buf, int st) {
        const int b0 = st * KS;
#pragma unroll
        for (int u = 0; u < T::A_CHUNKS; ++u) {
            const int c = tid + 256 * u;
            if (T::A_TOTAL % 256 == 0 || c < T::A_TOTAL) {
                const int row = c / (2 * KS), part = c % (2 * KS);
                *reinterpret_cast<u4v*>(buf + row * T::A_STRIDE + 16 * part) = ra[u];
            }
        }
        constexpr int BPARTS = T::WBYTES * KS / 16;
        uint8_t* bbuf = buf + T::A_BYTES;
#pragma unroll
        for (int u = 0; u < T::B_CHUNKS; ++u) {
            const int c = tid + 256 * u;
            if (T::B_TOTAL % 256 == 0 || c < T::B_TOTAL) {
                const int colx = c / BPARTS, part = c % BPARTS;
                *reinterpret_cast<u4v*>(bbuf + colx * T::B_STRIDE + 16 * part) = rb[u];
            }
        }
        // scales are stored block-major ([kb][row], [kb][column]) so that the
        // 32 lanes of a fragment read 32 consecutive words
        float* dxb = reinterpret_cast<float*>(buf + T::A_BYTES + T::B_BYTES);
#pragma unroll
        for (int u = 0; u < T::DX_ITEMS; ++u) {
            const int c = tid + 256 * u;
            if (c < T::BM * KS) dxb[(c % KS) * T::BM + c / KS] = b0 + c % KS < nb ? rdx[u] : 0.f;  // past K: zero
        }
        float* dwb = dxb + T::BM * KS;
#pragma unroll
        for (int u = 0; u < T::DW_ITEMS; ++u) {
            const int c = tid + 256 * u;
            if (c < NMAT * T::BN * KS) dwb[(c % KS) * (NMAT * T::BN) + c / KS] = Frag<F>::scale(rdw[u]);
        }
    };

    v16f acc[NMAT][TM][TN];
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[q][i][j][r] = 0.f;
    const v16i zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    v32f zf32;
#pragma unroll
    for (int r = 0; r < 32; ++r) zf32[r] = 0.f;

    // ---- one stage of math from an LDS buffer, blocks taken in pairs
    // (kb, kb + 1).  One v_mfma_f32_32x32x1_2b_f32 forms both blocks' scale
    // outer products d_x (x) d_w at once: its first block comes from lanes
    // 0-31 and lands in registers 0-15, its second from lanes 32-63 into
    // registers 16-31, each in the 32 x 32 result layout of the int8 MFMA.
    // So lane half lh simply reads block kb + lh's scale.  Per tile the
    // blocks are added in order, kb then kb + 1.
    static_assert(KS % 2 == 0, "blocks are taken in pairs");
    constexpr int NT = NMAT * TM * TN;
    auto compute = [&](const uint8_t* buf) {
        const uint8_t* abuf = buf;
        const uint8_t* bbuf = buf + T::A_BYTES;
        const float* dxb = reinterpret_cast<const float*>(buf + T::A_BYTES + T::B_BYTES);
        const float* dwb = dxb + T::BM * KS;
#pragma unroll 1
        for (int kb = 0; kb < KS; kb += 2) {
            v4i a[2][TM];
            float dx2[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * 32 * TM + 32 * i + li;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    a[h][i] = *reinterpret_cast<const v4i*>(abuf + row * T::A_STRIDE + 32 * (kb + h) + 16 * lh);
                dx2[i] = dxb[(kb + lh) * T::BM + row];
            }
            v4i bw[2][NMAT][TN];
            float dw2[NMAT][TN];
#pragma unroll
            for (int q = 0; q < NMAT; ++q) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int colx = q * T::BN + wn * 32 * TN + 32 * j + li;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint8_t* bp = bbuf + colx * T::B_STRIDE + T::WBYTES * (kb + h);
                        uint4 raw;
                        if constexpr (F == Fmt::Q8_0) raw = *reinterpret_cast<const uint4*>(bp + 16 * lh);
                        else raw = *reinterpret_cast<const uint4*>(bp);
                        bw[h][q][j] = Frag<F>::codes(raw, lh);
                    }
                    dw2[q][j] = dwb[(kb + lh) * (NMAT * T::BN) + colx];
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int q = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
                const v32f sc = __builtin_amdgcn_mfma_f32_32x32x1f32(dx2[i], dw2[q][j], zf32, 0, 0, 0);
                const v16i d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0][i], bw[0][q][j], zi, 0, 0, 0);
                const v16i d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[1][i], bw[1][q][j], zi, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[q][i][j][r] = __builtin_fmaf(static_cast<float>(d0[r]), sc[r], acc[q][i][j][r]);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[q][i][j][r] = __builtin_fmaf(static_cast<float>(d1[r]), sc[16 + r], acc[q][i][j][r]);
                // one tile's results live at a time
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    gload(0);
    lstore(lds, 0);
    __syncthreads();
    for (int st = 0; st < stages; ++st) {
        uint8_t* cur = lds + (st & 1) * T::STAGE;
        uint8_t* nxt = lds + ((st + 1) & 1) * T::STAGE;
        const bool more = st + 1 < stages;
        if (more) gload(st + 1);  // in flight during the math below
        compute(cur);
        if (more) lstore(nxt, st + 1);  // nxt was last read before the previous barrier
        __syncthreads();
    }

    // D layout: lane (li, lh), register r -> row 8(r/4) + 4 lh + r%4, column li
    const int m0 = mbase + wm * 32 * TM, n0 = nbase + wn * 32 * TN;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + 32 * j + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (row < M && col < N) {
                    const float v = MODE == Mode::SwiGLU ? swiglu_f32(acc[0][i][j][r], acc[NMAT - 1][i][j][r])
                                                         : acc[0][i][j][r];
                    y[static_cast<size_t>(row) * N + col] = v;
                }
            }
        }
    }
}

template <Fmt F, Mode MODE, int WGM, int WGN, int TM, int TN, int KS>
hipError_t launch(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                  const int8_t* xq, const float* xd, float* y, int M, int N, int K, hipStream_t stream) {
    using T = Tile<F, MODE, WGM, WGN, TM, TN, KS>;
    const int m_tiles = (M + T::BM - 1) / T::BM, n_tiles = (N + T::BN - 1) / T::BN;
    const long long total = static_cast<long long>(m_tiles) * n_tiles;
    if (total > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const size_t lds_bytes = 2 * static_cast<size_t>(T::STAGE);
    hipLaunchKernelGGL((qmm_mfma_kernel<F, MODE, WGM, WGN, TM, TN, KS>), dim3(static_cast<unsigned>(total)),
                       dim3(256), lds_bytes, stream, static_cast<const uint8_t*>(wa), sa,
                       static_cast<const uint8_t*>(wb), sb, xq, xd, y, M, N, K, m_tiles, n_tiles);
    return hipGetLastError();
}

// LDS-DMA variant of the kernel above, for K a multiple of four blocks and
// 16-byte aligned codes.  The gfx950 global_load_lds_dwordx4 copies each
// lane's 16 bytes straight from global memory into LDS (lane i of a wave
// instruction to byte 16 i of a 1 KB run), so a stage is loaded without
// staging registers, LDS stores or per-stage address arithmetic: every
// lane keeps one 32-bit offset per copy it issues, and the stage advances a
// uniform base pointer.  A copy writes 1 KB contiguously, so rows cannot be
// padded apart; instead the 16-byte chunks of a row are stored XOR-permuted
// by the row index, which spreads the fragment reads of 8 consecutive rows
// over distinct LDS banks.  Two statically separate stage buffers let the
// compiler see that the copies in flight never touch the buffer being read.
// The arithmetic is the one above, block by block in the same order, with
// the 4-bit factor 1/16 applied to the finished sums (a power of two).
typedef __attribute__((address_space(3))) void* lds_dst_t;
typedef const __attribute__((address_space(1))) void* glb_src_t;

// lane i: 16 (or 4) bytes from src into dst + 16 i (dst + 4 i)
__device__ __forceinline__ void lds_copy16(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds((glb_src_t)src, (lds_dst_t)dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds((glb_src_t)src, (lds_dst_t)dst, 4, 0, 0);
}
// wait for this wave's copies (vmcnt 0; expcnt and lgkmcnt left alone)
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <Fmt F, Mode MODE, int WGM, int WGN, int TM, int TN>
struct DmaTile {
    static constexpr int KS = 4;  // blocks per stage
    static constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    static constexpr int BM = 32 * TM * WGM;  // activation rows
    static constexpr int BN = 32 * TN * WGN;  // weight columns per matrix
    static constexpr int WB = F == Fmt::Q8_0 ? 32 : 16;  // weight bytes per block
    static constexpr int A_ROW = 32 * KS;  // 128: 8 chunks of 16 bytes
    static constexpr int B_ROW = WB * KS;  // 64 (4 chunks) or 128 (8 chunks)
    static constexpr int A_BYTES = BM * A_ROW;
    static constexpr int B_BYTES = NMAT * BN * B_ROW;
    static constexpr int DX_BYTES = (BM > 64 ? BM : 64) * KS * 4;  // fp32 [row][block], whole 64-row copies
    static constexpr int DW_BYTES = NMAT * BN * KS * 2;  // [column][block] fp16 bits
    static constexpr int B_OFF = A_BYTES, DX_OFF = B_OFF + B_BYTES, DW_OFF = DX_OFF + DX_BYTES;
    static constexpr int STAGE = DW_OFF + DW_BYTES;
    // wave copies per stage: 1 KB each for codes and activation scales,
    // 256 B (dword lanes) for weight scales
    static constexpr int A_OPS = A_BYTES / 1024, B_OPS = B_BYTES / 1024;
    static constexpr int DX_OPS = DX_BYTES / 1024, DW_OPS = DW_BYTES / 256;
    // per wave (the four waves take copies o = wave, wave + 4, ...; a wave
    // past the last copy repeats it: the same bytes to the same place)
    static constexpr int A_PW = (A_OPS + 3) / 4, B_PW = (B_OPS + 3) / 4;
    static constexpr int DX_PW = (DX_OPS + 3) / 4, DW_PW = (DW_OPS + 3) / 4;
    static constexpr int B_COLS = 1024 / B_ROW;  // weight columns per copy
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "whole 1 KB copies");
    static_assert(DX_BYTES % 1024 == 0 && DW_BYTES % 256 == 0, "whole copies");
    static_assert(KS == 4 && BM % 32 == 0, "activation-scale copies: one 16-byte row per lane");
    static_assert(BN % B_COLS == 0 && BN % 32 == 0, "a copy stays inside one matrix");
};

// Chunk permutation inside a stored row.  A rows and Q8_0 weight columns
// hold 8 chunks of 16 bytes, 4-bit weight columns 4 (one block each).  The
// permutation puts the chunks that 16 lanes reading 16 consecutive rows (or
// columns) fetch at once on 16 distinct 16-byte bank groups, and the chunks
// of any 8 consecutive rows on 8 distinct ones.
__device__ __forceinline__ int row_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }
template <Fmt F>
__device__ __forceinline__ int b_swizzle(int col) {
    return F == Fmt::Q8_0 ? row_swizzle(col) : (((col >> 1) ^ (col >> 3)) & 3);
}

template <Fmt F, Mode MODE, int WGM, int WGN, int TM, int TN>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(F == Fmt::Q4 && MODE == Mode::Plain ? 3 : 2)))
void qmm_mfma_dma(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, float* __restrict__ y,
    int M, int N, int K, int m_tiles, int n_tiles) {
    static_assert(WGM * WGN == 4, "four waves per workgroup");
    using T = DmaTile<F, MODE, WGM, WGN, TM, TN>;
    constexpr int NMAT = T::NMAT, KS = T::KS;
    __shared__ __align__(16) uint8_t lds0[T::STAGE];
    __shared__ __align__(16) uint8_t lds1[T::STAGE];

    const int total = m_tiles * n_tiles;
    int g = blockIdx.x;
    if ((total & 7) == 0) g = (g & 7) * (total >> 3) + (g >> 3);  // XCD-contiguous ranges
    const int mt = g % m_tiles, nt = g / m_tiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;
    const int wm = wave % WGM, wn = wave / WGM;
    const int mbase = mt * T::BM, nbase = nt * T::BN;
    const int nb = K / kBlock;
    const int stages = nb / KS;
    const uint32_t wrow = F == Fmt::Q8_0 ? static_cast<uint32_t>(K) : static_cast<uint32_t>(K) / 2;

    // ---- per-lane source offsets of this wave's copies (rows and columns
    // past the matrix repeat the last one: in bounds, never stored)
    uint32_t a_off[T::A_PW], b_off[T::B_PW], dx_off[T::DX_PW], dw_off[T::DW_PW];
#pragma unroll
    for (int u = 0; u < T::A_PW; ++u) {
        const int o = min(wave + 4 * u, T::A_OPS - 1);
        const int r = 8 * o + lane / 8, slot = lane % 8;
        const int c = slot ^ row_swizzle(r);  // logical 16-byte chunk of the row
        a_off[u] = static_cast<uint32_t>(min(mbase + r, M - 1)) * static_cast<uint32_t>(K) + 16u * c;
    }
#pragma unroll
    for (int u = 0; u < T::B_PW; ++u) {
        const int o = min(wave + 4 * u, T::B_OPS - 1);
        constexpr int CPC = T::B_ROW / 16;  // chunks per column
        const int colx = T::B_COLS * o + lane / CPC, slot = lane % CPC;
        const int c = slot ^ b_swizzle<F>(colx);
        b_off[u] = static_cast<uint32_t>(min(nbase + colx % T::BN, N - 1)) * wrow + 16u * c;
    }
#pragma unroll
    for (int u = 0; u < T::DX_PW; ++u) {
        // copy o: rows 64 o + lane, the stage's four scales of a row (16
        // bytes, one lane each): the copy unit pays per distinct row, so a
        // row per lane costs half of two 8-byte pieces per row.  A 32-row
        // panel fills half of its copy; the other lanes read clamped rows
        // (in bounds) into LDS that nothing reads.
        const int o = min(wave + 4 * u, T::DX_OPS - 1);
        const int r = 64 * o + lane;
        dx_off[u] = static_cast<uint32_t>(min(mbase + r, M - 1)) * static_cast<uint32_t>(nb);
    }
#pragma unroll
    for (int u = 0; u < T::DW_PW; ++u) {
        const int o = min(wave + 4 * u, T::DW_OPS - 1);
        const int colx = 32 * o + lane / 2, h = lane % 2;  // 64 lanes = 32 columns x 2 dwords
        dw_off[u] = static_cast<uint32_t>(min(nbase + colx % T::BN, N - 1)) * static_cast<uint32_t>(nb) + 2u * h;
    }
    // one stage: blocks [KS st, KS st + KS) of every row and column
    auto issue = [&](int st, uint8_t* buf) {
        const int b0 = st * KS;
        const int8_t* xs = xq + 32 * b0;
#pragma unroll
        for (int u = 0; u < T::A_PW; ++u) {
            const int o = min(wave + 4 * u, T::A_OPS - 1);
            lds_copy16(xs + a_off[u], buf + 1024 * o);
        }
#pragma unroll
        for (int u = 0; u < T::B_PW; ++u) {
            const int o = min(wave + 4 * u, T::B_OPS - 1);
            const uint8_t* ws = (NMAT == 2 && o * T::B_COLS >= T::BN ? wb : wa) + T::WB * b0;
            lds_copy16(ws + b_off[u], buf + T::B_OFF + 1024 * o);
        }
#pragma unroll
        for (int u = 0; u < T::DX_PW; ++u) {
            const int o = min(wave + 4 * u, T::DX_OPS - 1);
            lds_copy16(xd + b0 + dx_off[u], buf + T::DX_OFF + 1024 * o);
        }
#pragma unroll
        for (int u = 0; u < T::DW_PW; ++u) {
            const int o = min(wave + 4 * u, T::DW_OPS - 1);
            const uint16_t* ss = (NMAT == 2 && 32 * o >= T::BN ? sb : sa) + b0;
            lds_copy4(ss + dw_off[u], buf + T::DW_OFF + 256 * o);
        }
    };

    // ---- per-lane LDS read offsets (the chunk permutation depends only on
    // the lane: tile rows and columns start at multiples of 32)
    int a_rd[KS], b_rd[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        a_rd[k] = (wm * 32 * TM + li) * T::A_ROW + 16 * ((2 * k + lh) ^ row_swizzle(li));
        if constexpr (F == Fmt::Q8_0)
            b_rd[k] = T::B_OFF + (wn * 32 * TN + li) * T::B_ROW + 16 * ((2 * k + lh) ^ b_swizzle<F>(li));
        else
            b_rd[k] = T::B_OFF + (wn * 32 * TN + li) * T::B_ROW + 16 * (k ^ b_swizzle<F>(li));
    }
    // activation scale of (row, block kb + lh): word 4 row + kb + lh
    const int dx_rd = T::DX_OFF + 16 * (wm * 32 * TM + li) + 4 * lh;
    const int dw_rd = T::DW_OFF + (wn * 32 * TN + li) * (2 * KS) + 2 * lh;

    v16f acc[NMAT][TM][TN];
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[q][i][j][r] = 0.f;
    const v16i zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    v32f zf32;
#pragma unroll
    for (int r = 0; r < 32; ++r) zf32[r] = 0.f;

    // the math of one stage, blocks in pairs (kb, kb + 1): the scale outer
    // products of both come from one v_mfma_f32_32x32x1_2b_f32 (lane half lh
    // reads block kb + lh), then each tile adds block kb, then kb + 1
    constexpr int NT = NMAT * TM * TN;
    auto compute = [&](const uint8_t* buf) {
#pragma unroll
        for (int kb = 0; kb < KS; kb += 2) {
            v4i a[2][TM];
            float dx2[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    a[h][i] = *reinterpret_cast<const v4i*>(buf + a_rd[kb + h] + 32 * i * T::A_ROW);
                dx2[i] = *reinterpret_cast<const float*>(buf + dx_rd + 512 * i + 4 * kb);
            }
            v4i bw[2][NMAT][TN];
            float dw2[NMAT][TN];
#pragma unroll
            for (int q = 0; q < NMAT; ++q) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int cshift = q * T::BN + 32 * j;  // columns past this lane's first
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint4 raw = *reinterpret_cast<const uint4*>(buf + b_rd[kb + h] + cshift * T::B_ROW);
                        bw[h][q][j] = Frag<F>::codes(raw, lh);
                    }
                    dw2[q][j] = f16_bits_to_f32(
                        *reinterpret_cast<const uint16_t*>(buf + dw_rd + cshift * 2 * KS + 2 * kb));
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int q = t / (TM * TN), i = (t / TN) % TM, j = t % TN;
                const v32f sc = __builtin_amdgcn_mfma_f32_32x32x1f32(dx2[i], dw2[q][j], zf32, 0, 0, 0);
                const v16i d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0][i], bw[0][q][j], zi, 0, 0, 0);
                const v16i d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[1][i], bw[1][q][j], zi, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[q][i][j][r] = __builtin_fmaf(static_cast<float>(d0[r]), sc[r], acc[q][i][j][r]);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[q][i][j][r] = __builtin_fmaf(static_cast<float>(d1[r]), sc[16 + r], acc[q][i][j][r]);
                __builtin_amdgcn_sched_barrier(0);  // one tile's results live at a time
            }
        }
    };

    // ---- pipeline: the copies of stage st + 1 fly while stage st is
    // multiplied; one barrier per stage (after it, every wave's copies of
    // the stage have landed and every wave is done with the other buffer).
    // The last pair's second copy repeats the last stage (in bounds, unused).
    issue(0, lds0);
    int st = 0;
    for (; st + 1 < stages; st += 2) {
        wait_copies();
        __syncthreads();
        issue(st + 1, lds1);
        __builtin_amdgcn_sched_barrier(0);
        compute(lds0);
        wait_copies();
        __syncthreads();
        issue(min(st + 2, stages - 1), lds0);
        __builtin_amdgcn_sched_barrier(0);
        compute(lds1);
    }
    wait_copies();
    if (st < stages) {  // an odd stage count: the last stage is in lds0
        __syncthreads();
        compute(lds0);
    }

    // D layout: lane (li, lh), register r -> row 8(r/4) + 4 lh + r%4, column li
    constexpr float kOut = F == Fmt::Q4 ? 0.0625f : 1.0f;  // 4-bit codes carry 16
    const int m0 = mbase + wm * 32 * TM, n0 = nbase + wn * 32 * TN;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + 32 * j + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (row < M && col < N) {
                    const float v = MODE == Mode::SwiGLU
                                        ? swiglu_f32(acc[0][i][j][r] * kOut, acc[NMAT - 1][i][j][r] * kOut)
                                        : acc[0][i][j][r] * kOut;
                    y[static_cast<size_t>(row) * N + col] = v;
                }
            }
        }
    }
}

template <Fmt F, Mode MODE, int WGM, int WGN, int TM, int TN>
hipError_t launch_dma(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                      const int8_t* xq, const float* xd, float* y, int M, int N, int K, hipStream_t stream) {
    using T = DmaTile<F, MODE, WGM, WGN, TM, TN>;
    const int m_tiles = (M + T::BM - 1) / T::BM, n_tiles = (N + T::BN - 1) / T::BN;
    const long long total = static_cast<long long>(m_tiles) * n_tiles;
    if (total > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((qmm_mfma_dma<F, MODE, WGM, WGN, TM, TN>), dim3(static_cast<unsigned>(total)), dim3(256),
                       0, stream, static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb, xq,
                       xd, y, M, N, K, m_tiles, n_tiles);
    return hipGetLastError();
}

// The LDS-DMA kernel needs whole stages of four blocks, 16-byte aligned
// code rows (K is a multiple of 32, so only the base pointers matter) and
// activation-scale rows (K / 32 is then a multiple of 4), 4-byte aligned
// weight-scale pairs, and 32-bit source offsets.
bool dma_eligible(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                  const int8_t* xq, const float* xd, long long M, long long N, long long K) {
    auto al = [](const void* p, uintptr_t a) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % a == 0; };
    return (K / kBlock) % 4 == 0 && al(wa, 16) && al(wb, 16) && al(xq, 16) && al(sa, 4) && al(sb, 4) &&
           al(xd, 16) && M * K < (1LL << 31) && N * K < (1LL << 31);
}

// Split-K kernel for short panels (up to 64 rows) whose output holds too
// few 32 x 32 tiles to fill the chip (the pp32 projections: 28 to 152
// column tiles).  A workgroup of NW waves owns one 32-column tile (per
// weight matrix) and all TM x 32 rows, and walks K in stages of KC blocks:
// the whole workgroup loads a stage with coalesced 16-byte reads along the
// rows (full cache lines; fragment-shaped gathers of 32 rows x 32 bytes
// cost the address unit a line per lane pair), stores it to LDS, and each
// wave multiplies its KC / NW blocks of the stage.  Each block is formed
// whole on the matrix core (exact int32) and scaled into the wave's fp32
// accumulators; the NW partial tiles are then added in wave order through
// LDS.  The next stage's loads are in flight during the current math.
template <Fmt F, Mode MODE, int TM, int NW>
struct SplitTile {
    static constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    static constexpr int KC = 16;                       // blocks per stage
    static constexpr int BPW = KC / NW;                 // blocks per wave per stage
    static constexpr int NT = 64 * NW;                  // threads
    static constexpr int WBYTES = F == Fmt::Q8_0 ? 32 : 16;
    static constexpr int ROWS = 32 * TM;
    static constexpr int A_STRIDE = 32 * KC + 16;
    static constexpr int B_STRIDE = WBYTES * KC + 16;
    static constexpr int A_BYTES = ROWS * A_STRIDE;
    static constexpr int B_BYTES = NMAT * 32 * B_STRIDE;
    static constexpr int DX_BYTES = ROWS * KC * 4;
    static constexpr int DW_BYTES = NMAT * 32 * KC * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES + DX_BYTES + DW_BYTES;
    static constexpr int RED = NW * NMAT * TM * 16 * 64 * 4;
    static constexpr int LDS = 2 * STAGE > RED ? 2 * STAGE : RED;
    static constexpr int A_TOTAL = ROWS * 2 * KC;               // 16-byte parts
    static constexpr int B_TOTAL = NMAT * 32 * (WBYTES * KC / 16);
    static constexpr int A_CHUNKS = (A_TOTAL + NT - 1) / NT;
    static constexpr int B_CHUNKS = (B_TOTAL + NT - 1) / NT;
    static constexpr int DX_ITEMS = (ROWS * KC + NT - 1) / NT;
    static constexpr int DW_ITEMS = (NMAT * 32 * KC + NT - 1) / NT;
    static_assert(KC % NW == 0, "whole blocks per wave");
};

template <Fmt F, Mode MODE, int TM, int NW>
__global__ __launch_bounds__(64 * NW) void qmm_mfma_splitk(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, float* __restrict__ y,
    int M, int N, int K) {
    using T = SplitTile<F, MODE, TM, NW>;
    constexpr int NMAT = T::NMAT, KC = T::KC, NT = T::NT;
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lh = lane >> 5;
    const int nb = K / kBlock;
    const int stages = (nb + KC - 1) / KC;
    const int nbase = static_cast<int>(blockIdx.x) * 32;
    const size_t wrow = F == Fmt::Q8_0 ? static_cast<size_t>(K) : static_cast<size_t>(K) / 2;

    // ---- global -> registers (every load in bounds: rows, columns and
    // blocks clamped; blocks past K get a zero activation scale at the store)
    u4v ra[T::A_CHUNKS], rb[T::B_CHUNKS];
    float rdx[T::DX_ITEMS];
    uint16_t rdw[T::DW_ITEMS];
    auto gload = [&](int st) {
        const int b0 = st * KC;
#pragma unroll
        for (int u = 0; u < T::A_CHUNKS; ++u) {
            const int c = min(tid + NT * u, T::A_TOTAL - 1);
            const int row = c / (2 * KC), part = c % (2 * KC);
            const int r = min(row, M - 1);
            const int blk = min(b0 + part / 2, nb - 1);
            ra[u] = *reinterpret_cast<const u4v*>(xq + static_cast<size_t>(r) * K + 32 * blk + 16 * (part & 1));
        }
        constexpr int BPARTS = T::WBYTES * KC / 16;
        constexpr int BPB = T::WBYTES / 16;
#pragma unroll
        for (int u = 0; u < T::B_CHUNKS; ++u) {
            const int c = min(tid + NT * u, T::B_TOTAL - 1);
            const int colx = c / BPARTS, part = c % BPARTS;
            const int q = colx / 32, col = colx % 32;
            const int cc = min(nbase + col, N - 1);
            const int blk = min(b0 + part / BPB, nb - 1);
            const uint8_t* w = (NMAT == 2 && q == 1) ? wb : wa;
            rb[u] = *reinterpret_cast<const u4v*>(w + static_cast<size_t>(cc) * wrow + T::WBYTES * blk + 16 * (part % BPB));
        }
#pragma unroll
        for (int u = 0; u < T::DX_ITEMS; ++u) {
            const int c = min(tid + NT * u, T::ROWS * KC - 1);
            const int row = c / KC, kb = c % KC;
            rdx[u] = xd[static_cast<size_t>(min(row, M - 1)) * nb + min(b0 + kb, nb - 1)];
        }
#pragma unroll
        for (int u = 0; u < T::DW_ITEMS; ++u) {
            const int c = min(tid + NT * u, NMAT * 32 * KC - 1);
            const int colx = c / KC, kb = c % KC;
            const int q = colx / 32, col = colx % 32;
            const uint16_t* sc = (NMAT == 2 && q == 1) ? sb : sa;
            rdw[u] = sc[static_cast<size_t>(min(nbase + col, N - 1)) * nb + min(b0 + kb, nb - 1)];
        }
    };
    auto lstore = [&](uint8_t* buf, int st) {
        const int b0 = st * KC;
#pragma unroll
        for (int u = 0; u < T::A_CHUNKS; ++u) {
            const int c = tid + NT * u;
            if (T::A_TOTAL % NT == 0 || c < T::A_TOTAL) {
                const int row = c / (2 * KC), part = c % (2 * KC);
                *reinterpret_cast<u4v*>(buf + row * T::A_STRIDE + 16 * part) = ra[u];
            }
        }
        constexpr int BPARTS = T::WBYTES * KC / 16;
        uint8_t* bbuf = buf + T::A_BYTES;
#pragma unroll
        for (int u = 0; u < T::B_CHUNKS; ++u) {
            const int c = tid + NT * u;
            if (T::B_TOTAL % NT == 0 || c < T::B_TOTAL) {
                const int colx = c / BPARTS, part = c % BPARTS;
                *reinterpret_cast<u4v*>(bbuf + colx * T::B_STRIDE + 16 * part) = rb[u];
            }
        }
        // scales block-major ([kb][row], [kb][column]): a fragment's 32 lanes
        // read 32 consecutive words
        float* dxb = reinterpret_cast<float*>(buf + T::A_BYTES + T::B_BYTES);
#pragma unroll
        for (int u = 0; u < T::DX_ITEMS; ++u) {
            const int c = tid + NT * u;
            if (c < T::ROWS * KC) dxb[(c % KC) * T::ROWS + c / KC] = b0 + c % KC < nb ? rdx[u] : 0.f;
        }
        float* dwb = dxb + T::ROWS * KC;
#pragma unroll
        for (int u = 0; u < T::DW_ITEMS; ++u) {
            const int c = tid + NT * u;
            if (c < NMAT * 32 * KC) dwb[(c % KC) * (NMAT * 32) + c / KC] = Frag<F>::scale(rdw[u]);
        }
    };

    v16f acc[NMAT][TM];
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[q][i][r] = 0.f;
    const v16i zi = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const v16f zf = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // ---- this wave's blocks of a stage: kb = BPW * wave + j
    auto compute = [&](const uint8_t* buf) {
        const uint8_t* abuf = buf;
        const uint8_t* bbuf = buf + T::A_BYTES;
        const float* dxb = reinterpret_cast<const float*>(buf + T::A_BYTES + T::B_BYTES);
        const float* dwb = dxb + T::ROWS * KC;
#pragma unroll 1
        for (int j = 0; j < T::BPW; ++j) {
            const int kb = T::BPW * wave + j;
            v4i a[TM];
            float dx[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = 32 * i + li;
                a[i] = *reinterpret_cast<const v4i*>(abuf + row * T::A_STRIDE + 32 * kb + 16 * lh);
                const float v = dxb[kb * T::ROWS + row];
                dx[i] = lh == 0 ? v : 0.f;  // k = 1 half of the rank-1 product is zero
            }
#pragma unroll
            for (int q = 0; q < NMAT; ++q) {
                const int colx = 32 * q + li;
                const uint8_t* bp = bbuf + colx * T::B_STRIDE + T::WBYTES * kb;
                uint4 raw;
                if constexpr (F == Fmt::Q8_0) raw = *reinterpret_cast<const uint4*>(bp + 16 * lh);
                else raw = *reinterpret_cast<const uint4*>(bp);
                const v4i bw = Frag<F>::codes(raw, lh);
                const float v = dwb[kb * (NMAT * 32) + colx];
                const float dw = lh == 0 ? v : 0.f;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const v16i dot = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bw, zi, 0, 0, 0);
                    const v16f sc = __builtin_amdgcn_mfma_f32_32x32x2f32(dx[i], dw, zf, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[q][i][r] = __builtin_fmaf(static_cast<float>(dot[r]), sc[r], acc[q][i][r]);
                    // one tile's results live at a time (no hoisting of the next MFMAs)
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    gload(0);
    lstore(lds, 0);
    __syncthreads();
    for (int st = 0; st < stages; ++st) {
        uint8_t* cur = lds + (st & 1) * T::STAGE;
        uint8_t* nxt = lds + ((st + 1) & 1) * T::STAGE;
        const bool more = st + 1 < stages;
        if (more) gload(st + 1);  // in flight during the math below
        compute(cur);
        if (more) lstore(nxt, st + 1);  // nxt was last read before the previous barrier
        __syncthreads();
    }

    // partial tiles -> LDS as [wave][q][i][r][lane] (the stages are done:
    // the barrier above ends every read of them), then a fixed wave-order sum
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                red[(((wave * NMAT + q) * TM + i) * 16 + r) * 64 + lane] = acc[q][i][r];
    __syncthreads();
    constexpr int ELEMS = TM * 16 * 64;  // per matrix: (i, r, lane)
    for (int e = tid; e < ELEMS; e += NT) {
        const int i = e / (16 * 64), r = (e / 64) % 16, l = e % 64;
        float v[NMAT];
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            float sum = 0.f;
            for (int w = 0; w < NW; ++w) sum += red[(((w * NMAT + q) * TM + i) * 16 + r) * 64 + l];
            v[q] = sum;
        }
        // D layout: lane (l % 32, l / 32), register r -> row 8(r/4) + 4(l/32) + r%4, column l % 32
        const int row = 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        const int c = nbase + (l & 31);
        if (row < M && c < N)
            y[static_cast<size_t>(row) * N + c] = MODE == Mode::SwiGLU ? swiglu_f32(v[0], v[NMAT - 1]) : v[0];
    }
}

template <Fmt F, Mode MODE, int TM, int NW>
hipError_t launch_splitk(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                         const int8_t* xq, const float* xd, float* y, int M, int N, int K,
                         hipStream_t stream) {
    using T = SplitTile<F, MODE, TM, NW>;
    const unsigned tiles = static_cast<unsigned>((N + 31) / 32);
    hipLaunchKernelGGL((qmm_mfma_splitk<F, MODE, TM, NW>), dim3(tiles), dim3(64 * NW),
                       static_cast<size_t>(T::LDS), stream, static_cast<const uint8_t*>(wa), sa,
                       static_cast<const uint8_t*>(wb), sb, xq, xd, y, M, N, K);
    return hipGetLastError();
}

template <Fmt F, Mode MODE>
hipError_t dispatch_splitk(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                           const int8_t* xq, const float* xd, float* y, int M, int N, int K,
                           hipStream_t stream) {
    const int nw = static_cast<int>(plan::splitk_waves(F, M));
    if (M <= 32) {
        if constexpr (F == Fmt::Q8_0)
            if (nw == 16) return launch_splitk<F, MODE, 1, 16>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        return launch_splitk<F, MODE, 1, 8>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
    }
    return launch_splitk<F, MODE, 2, 8>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
}

}  // namespace

hipError_t launch_qmm_q8act_mfma(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa,
                                 const void* wb, const uint16_t* sb, const int8_t* xq,
                                 const float* xd, float* y, int64_t M, int64_t N, int64_t K,
                                 hipStream_t stream) {
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    // Panels of up to 64 rows whose output is a few hundred 32 x 32 tiles:
    // split K across the waves of a workgroup (shape rule of M, N, K only).
    if (plan::q8act_plan(fmt, M, N, K, device_cus()).kernel == plan::Q8Kernel::SplitK) {
        if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
            return dispatch_splitk<Fmt::Q8_0, Mode::Plain>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        if (fmt == Fmt::Q4 && mode == Mode::Plain)
            return dispatch_splitk<Fmt::Q4, Mode::Plain>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
            return dispatch_splitk<Fmt::Q4, Mode::SwiGLU>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        return hipErrorInvalidValue;
    }
    // Panels of up to 32 rows: one row of four waves across N, one 32 x 32
    // tile each (small N still yields enough workgroups); larger panels:
    // waves of 64 x 32 tiles per matrix, 2 x 2 of them (128 x 64 per
    // workgroup), or 1 x 4 (64 x 128) for the plain 4-bit product.
    // Whole stages of four blocks and aligned rows: the LDS-DMA kernel.
    if (dma_eligible(wa, sa, wb, sb, xq, xd, M, N, K)) {
        if (fmt == Fmt::Q8_0 && mode == Mode::Plain) {
            if (m <= 32) return launch_dma<Fmt::Q8_0, Mode::Plain, 1, 4, 1, 1>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
            return launch_dma<Fmt::Q8_0, Mode::Plain, 2, 2, 2, 1>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        }
        if (fmt == Fmt::Q4 && mode == Mode::Plain) {
            if (m <= 32) return launch_dma<Fmt::Q4, Mode::Plain, 1, 4, 1, 1>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
            // 64 x 128 per workgroup: a fifth fewer copied bytes per tile-block than
            // 128 x 64 (4-bit weight rows are the cheaper operand), about 1% faster settled
            return launch_dma<Fmt::Q4, Mode::Plain, 1, 4, 2, 1>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        }
        if (fmt == Fmt::Q4 && mode == Mode::SwiGLU) {
            if (m <= 32) return launch_dma<Fmt::Q4, Mode::SwiGLU, 1, 4, 1, 1>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
            return launch_dma<Fmt::Q4, Mode::SwiGLU, 2, 2, 2, 1>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        }
        return hipErrorInvalidValue;
    }
    if (fmt == Fmt::Q8_0 && mode == Mode::Plain) {
        if (m <= 32) return launch<Fmt::Q8_0, Mode::Plain, 1, 4, 1, 1, 4>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        return launch<Fmt::Q8_0, Mode::Plain, 2, 2, 2, 1, 2>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
    }
    if (fmt == Fmt::Q4 && mode == Mode::Plain) {
        if (m <= 32) return launch<Fmt::Q4, Mode::Plain, 1, 4, 1, 1, 4>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        return launch<Fmt::Q4, Mode::Plain, 2, 2, 2, 1, 4>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
    }
    if (fmt == Fmt::Q4 && mode == Mode::SwiGLU) {
        if (m <= 32) return launch<Fmt::Q4, Mode::SwiGLU, 1, 4, 1, 1, 4>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        return launch<Fmt::Q4, Mode::SwiGLU, 2, 2, 2, 1, 4>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qbd
