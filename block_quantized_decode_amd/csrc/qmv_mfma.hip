// Block-quantized weights x fp32 activation panels (M = 2 .. 16) on the
// gfx950 matrix cores.
//
// At M = 8 the 4-bit gate/up SwiGLU consumer (LSE v0.4.16 release page,
// "Combined M8 Q4 gate/up execution") and the M8 down projection that the
// same page keeps on the matrix cores ("Retained optimizations and
// compatibility") are dense contractions: every weight meets M activation
// rows.  On the VALU each code then costs a conversion plus M fp32 FMAs,
// which bounds those kernels by FMA issue, far below the HBM rate.  Here
// the products run on v_mfma_f32_16x16x32_bf16 with no loss of exactness:
// - a code (int8, or 16 (q - 8) for a 4-bit block) has at most 8
//   significant bits, so it is exact in bf16;
// - an fp32 activation is split into three bf16 parts whose sum is exactly
//   the activation: the top 8 significant bits (truncation), the next 8 of
//   the remainder, and what is left, which has at most 8 bits;
// - a bf16 x bf16 product is exact in fp32, and the matrix core
//   accumulates in fp32, so each block dot is an fp32 sum of the exact
//   terms code * x, as in the VALU kernels, only in another order; the
//   block scale then multiplies it into an fp32 accumulator.
// Activations whose parts fall below the normal range (|x| under about
// 2^-110) or overflow bf16 (|x| above its largest finite value) are
// outside what this split represents exactly.
//
// MFMA operands (16 x 16 x 32): A is the activation panel (row m = lane % 16,
// K slots 8 * (lane / 16) + j), B the weights (column n = lane % 16, same K
// slots), D lane l holds rows 4 * (l / 16) + i of column l % 16.  A block of
// 32 codes is one MFMA K step, so the block scale of row n multiplies one
// whole D column.  The K order inside a block is free as long as A and B
// agree; it follows the byte order of the weight blocks (see MFrag).
//
// Panels of at most 8 rows use the 8 spare A rows: rows 0-7 carry the high
// parts and rows 8-15 the middle parts in one MFMA, the low parts ride in a
// second one, and the two halves of D are added once, after the K loop.
//
// Work split: one workgroup owns a run of 16-row weight tiles (NT at most)
// for both matrices of the SwiGLU mode; its NW waves split K by groups of
// blocks (group g of wave w: g = w, w + NW, ...), so each wave converts a
// group's activations once for all of its tiles.  Each 16-byte lane load
// reads a 64-byte run of one row (4 blocks of 4-bit codes, 2 of int8), and
// v_permlane16/32_swap turn the four loads of a row into the four K slots
// of the MFMA operand.  The scale rows of the tiles are contiguous in
// memory and are copied to LDS once: read per row from global memory, a
// few scales per load, they cost several times their bytes.  Partial sums
// meet in LDS at the end and are added in wave order, so every output has
// one fixed summation order and the plain and SwiGLU modes give the same
// projection bits.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace qbd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4_t a, const u32x4_t b, const f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two floats whose low 16 bits are zero, as one bf16 pair (u low, v high).
__device__ __forceinline__ uint32_t pack_bf16(float u, float v) {
    return __builtin_amdgcn_perm(__float_as_uint(v), __float_as_uint(u), 0x07060302u);
}

// x truncated to its top 8 significant bits (a bf16 value, as fp32).
__device__ __forceinline__ float top8(float x) {
    return __uint_as_float(__float_as_uint(x) & 0xFFFF0000u);
}

// swap32(a, b): a' = [a.lo32, b.lo32], b' = [a.hi32, b.hi32] (16-lane rows
// a0 a1 b0 b1 and a2 a3 b2 b3); swap16(a, b): a' = [a0 b0 a2 b2],
// b' = [a1 b1 a3 b3].
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

template <Fmt F> struct MFrag;

// 4-bit blocks (16 bytes each; byte j: code j low, code j + 16 high).  A
// lane load of row n, lane group j, reads block 4 * group + j whole; the
// exchange leaves in lane group g, register s, dword g of block s: codes
// 4g .. 4g + 3 (low nibbles) and 16 + 4g .. 16 + 4g + 3 (high nibbles).
template <> struct MFrag<Fmt::Q4> {
    static constexpr int kBlocks = 4;           // blocks per lane load
    static constexpr float kOutScale = 0.0625f;  // codes carry a factor 16
    __device__ static size_t row_bytes(int K) { return static_cast<size_t>(K) / 2; }
    __device__ static int chunk(int grp, int lg, int nb) { return min(kBlocks * grp + lg, nb - 1); }
    __device__ static void exchange(u32x4_t& w) {
        uint32_t a = w[0], b = w[1], c = w[2], d = w[3];
        swap32(a, c);
        swap32(b, d);
        swap16(a, b);
        swap16(c, d);
        w[0] = a; w[1] = b; w[2] = c; w[3] = d;
    }
    // block s of the group: 8 codes 16 (q - 8) as bf16, slots 0-3 = low
    // nibbles, 4-7 = high nibbles
    __device__ static u32x4_t codes(const u32x4_t& w, int s) {
        const uint32_t lo = q4x16_lo(w[s]), hi = q4x16_hi(w[s]);
        u32x4_t r;
        r[0] = pack_bf16(sbyte_f32<0>(lo), sbyte_f32<1>(lo));
        r[1] = pack_bf16(sbyte_f32<2>(lo), sbyte_f32<3>(lo));
        r[2] = pack_bf16(sbyte_f32<0>(hi), sbyte_f32<1>(hi));
        r[3] = pack_bf16(sbyte_f32<2>(hi), sbyte_f32<3>(hi));
        return r;
    }
    // columns of slots 0-3 and 4-7 inside a block, for lane group g
    __device__ static int col0(int g) { return 4 * g; }
    __device__ static int col1(int g) { return 16 + 4 * g; }
};

// Q8_0 blocks (32 int8 codes).  A lane load of row n, lane group j, reads
// bytes 16 j .. 16 j + 15 of a two-block run; the exchange leaves in lane
// group g, registers 2s and 2s + 1, bytes 8g .. 8g + 7 of block s.
template <> struct MFrag<Fmt::Q8_0> {
    static constexpr int kBlocks = 2;
    static constexpr float kOutScale = 1.0f;
    __device__ static size_t row_bytes(int K) { return static_cast<size_t>(K); }
    __device__ static int chunk(int grp, int lg, int nb) { return min(4 * grp + lg, 2 * nb - 1); }
    __device__ static void exchange(u32x4_t& w) {
        uint32_t a = w[0], b = w[1], c = w[2], d = w[3];
        swap16(a, c);
        swap16(b, d);
        swap32(a, c);
        swap32(b, d);
        w[0] = a; w[1] = b; w[2] = c; w[3] = d;
    }
    __device__ static u32x4_t codes(const u32x4_t& w, int s) {
        const uint32_t p = w[2 * s], q = w[2 * s + 1];
        u32x4_t r;
        r[0] = pack_bf16(sbyte_f32<0>(p), sbyte_f32<1>(p));
        r[1] = pack_bf16(sbyte_f32<2>(p), sbyte_f32<3>(p));
        r[2] = pack_bf16(sbyte_f32<0>(q), sbyte_f32<1>(q));
        r[3] = pack_bf16(sbyte_f32<2>(q), sbyte_f32<3>(q));
        return r;
    }
    __device__ static int col0(int g) { return 8 * g; }
    __device__ static int col1(int g) { return 8 * g + 4; }
};

// A operands of one block: NA bf16 vectors (2 for panels of at most 8 rows,
// 3 for 16).
template <int MT>
struct AOps {
    static constexpr int NA = MT <= 8 ? 2 : 3;
    u32x4_t a[NA];
};

// Split 8 activations into the operands of one block.  MT <= 8: a[0] holds
// the high parts (A rows 0-7) or the middle parts (rows 8-15), a[1] the low
// parts (rows 0-7) or zero.  MT = 16: a[0] high, a[1] middle, a[2] low.
template <int MT>
__device__ __forceinline__ void split_x(const float (&x)[8], bool upper, AOps<MT>& op) {
    float h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = top8(x[i]);
        const float r = x[i] - h[i];  // exact: the low 16 significant bits
        m[i] = top8(r);
        l[i] = r - m[i];              // exact, at most 8 significant bits
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t ph = pack_bf16(h[2 * p], h[2 * p + 1]);
        const uint32_t pm = pack_bf16(m[2 * p], m[2 * p + 1]);
        const uint32_t pl = pack_bf16(l[2 * p], l[2 * p + 1]);
        if constexpr (MT <= 8) {
            op.a[0][p] = upper ? pm : ph;
            op.a[1][p] = upper ? 0u : pl;
        } else {
            op.a[0][p] = ph;
            op.a[1][p] = pm;
            op.a[2][p] = pl;
        }
    }
}

template <int MT>
__device__ __forceinline__ f32x4_t block_dot(const AOps<MT>& op, const u32x4_t b) {
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MT <= 8) {
        return mfma_bf16(op.a[0], b, mfma_bf16(op.a[1], b, z));
    } else {
        return mfma_bf16(op.a[0], b, mfma_bf16(op.a[1], b, mfma_bf16(op.a[2], b, z)));
    }
}

// Padded length (uint16 entries) of a scale row in LDS: a multiple of 4, so
// the 4 scales of a 4-bit group are one aligned 8-byte read, with the rows
// of a tile on distinct LDS banks.
__host__ __device__ inline int scale_row_lds(int nb) { return static_cast<int>(plan::mfma_scale_row(nb)); }

// Copy the scale rows of a workgroup's tile slots to LDS: row r of matrix q
// comes from global row row_of(r).  Each wave copies whole rows, U at a
// time (all loads of a pass issued before its stores), its lanes taking the
// 8-byte pieces of a row (a lane past the end of a row repeats the row's
// last piece, the same bytes to the same place); rows whose scales are not
// 8-byte aligned go entry by entry.  No index here divides by a run-time
// value.
template <int NMAT, int ROWS, int NW, typename RowOf>
__device__ __forceinline__ void copy_scales(uint16_t* sst, int srl, const uint16_t* const (&sm)[2], int nb,
                                            RowOf row_of) {
    constexpr int NR = NMAT * ROWS;  // rows of all matrices
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool wide = nb % 4 == 0 && reinterpret_cast<uintptr_t>(sm[0]) % 8 == 0 &&
                      reinterpret_cast<uintptr_t>(sm[NMAT - 1]) % 8 == 0;
    if (wide) {
        constexpr int U = 8;
        const int per_row = nb / 4;
        for (int j0 = 0; j0 < per_row; j0 += 64) {
            const int j = min(j0 + lane, per_row - 1);
            for (int r0 = wave; r0 < NR; r0 += U * NW) {
                uint2 v[U];
#pragma unroll
                for (int k = 0; k < U; ++k) {
                    const int r = min(r0 + k * NW, NR - 1);
                    v[k] = *reinterpret_cast<const uint2*>(sm[r / ROWS] + static_cast<size_t>(row_of(r % ROWS)) * nb + 4 * j);
                }
#pragma unroll
                for (int k = 0; k < U; ++k) {
                    const int r = min(r0 + k * NW, NR - 1);
                    *reinterpret_cast<uint2*>(sst + r * srl + 4 * j) = v[k];
                }
            }
        }
    } else {
        // rows of a length that is not a multiple of 4: the entries up to the
        // next multiple of 4 are zeros, the scales of the blocks past K that a
        // last, partial group reads (so they add exactly zero)
        const int padded = (nb + 3) / 4 * 4;
        for (int r = wave; r < NR; r += NW) {
            const uint16_t* src = sm[r / ROWS] + static_cast<size_t>(row_of(r % ROWS)) * nb;
            for (int b = lane; b < padded; b += 64) sst[r * srl + b] = b < nb ? src[b] : uint16_t{0};
        }
    }
}

template <Fmt F, Mode MODE, int MT, int NT, int NW>
__global__ __launch_bounds__(NW * 64) void qmv_f32_mfma(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int M, int N, int K) {
    using G = MFrag<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int BPG = G::kBlocks;
    constexpr int MTO = MT <= 8 ? 8 : 16;  // output rows per tile
    constexpr int ROWS = NT * 16;          // tile rows of the workgroup
    extern __shared__ __align__(16) uint8_t lds[];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int nb = K / kBlock;
    const int ngroups = (nb + BPG - 1) / BPG;
    const size_t rbytes = G::row_bytes(K);
    const uint8_t* const wm[2] = {wa, wb};
    const uint16_t* const sm[2] = {sa, sb};

    // this workgroup's tiles: [tb, te), at most NT; slots past te repeat
    // the last tile (loads stay in bounds, results are not stored)
    const int ntiles = (N + 15) / 16;
    const int tb = static_cast<int>(static_cast<int64_t>(blockIdx.x) * ntiles / gridDim.x);
    const int te = static_cast<int>(static_cast<int64_t>(blockIdx.x + 1) * ntiles / gridDim.x);
    auto tile_row = [&](int r) {  // weight row of tile slot row r
        return min((tb + min(r / 16, te - tb - 1)) * 16 + r % 16, N - 1);
    };
    size_t wrow[NT];  // byte offset of this lane's weight row, per tile
#pragma unroll
    for (int t = 0; t < NT; ++t) wrow[t] = static_cast<size_t>(tile_row(t * 16 + ln)) * rbytes;


    // this lane's activation row and the part of it that it carries; rows
    // at or past M repeat row M - 1 (finite values whose products land in
    // rows of D that are never stored)
    const int mrow = MT <= 8 ? (ln & 7) : ln;
    const bool upper = MT <= 8 && ln >= 8;
    const float* xrow = x + static_cast<size_t>(min(mrow, M - 1)) * K;

    // This lane's weight row per tile and its x slices are held for one
    // group at a time; each is refilled with the next group's data as soon
    // as it has been used, so the loads of a group are in flight while the
    // rest of the current group is multiplied (loads past the last group
    // repeat it: in bounds, unused).
    u32x4_t wv[NT][NMAT];
    float xv[BPG][8];
    auto load_w = [&](int t, int q, int grp) {
        const int c = G::chunk(grp, lg, nb);
        // a plain (temporal) load: the other half of each 128-byte line is
        // the neighbouring group, read by the next wave of this workgroup
        wv[t][q] = *reinterpret_cast<const u32x4_t*>(wm[q] + wrow[t] + static_cast<size_t>(c) * 16);
    };
    auto load_x = [&](int grp) {
#pragma unroll
        for (int s = 0; s < BPG; ++s) {
            const int b = min(grp * BPG + s, nb - 1);
            const float4 v0 = *reinterpret_cast<const float4*>(xrow + b * kBlock + G::col0(lg));
            const float4 v1 = *reinterpret_cast<const float4*>(xrow + b * kBlock + G::col1(lg));
            xv[s][0] = v0.x; xv[s][1] = v0.y; xv[s][2] = v0.z; xv[s][3] = v0.w;
            xv[s][4] = v1.x; xv[s][5] = v1.y; xv[s][6] = v1.z; xv[s][7] = v1.w;
        }
    };

    float acc[NT][NMAT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][q][i] = 0.f;

    // groups of this wave: wave, wave + NW, ...  A prefetch has no user in
    // its own iteration, so the scheduler would sink it to the end of the
    // loop body; a scheduling barrier after it keeps it where it is issued
    // (and keeps the next tile's arithmetic, which would otherwise be
    // hoisted with its waits, below its own prefetch).
    constexpr int kPinLoads = 0;
    const int last = ngroups - 1;
    // first group, in the order the loop body issues its prefetches (the
    // wait counts at the top of the loop follow the order of the loads);
    // issued before the scale rows are copied, so both are in flight at once
    load_x(min(wave, last));
    __builtin_amdgcn_sched_barrier(kPinLoads);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            load_w(t, q, min(wave, last));
            __builtin_amdgcn_sched_barrier(kPinLoads);
        }

    // the scale rows of the tiles, once (a last, partial group reads the
    // zero entries just past nb)
    const int srl = scale_row_lds(nb);
    uint16_t* const sst = reinterpret_cast<uint16_t*>(lds);
    copy_scales<NMAT, ROWS, NW>(sst, srl, sm, nb, tile_row);
    __syncthreads();
    for (int grp = wave; grp < ngroups; grp += NW) {
        const int nxt = min(grp + NW, last);
        AOps<MT> op[BPG];
#pragma unroll
        for (int s = 0; s < BPG; ++s) split_x<MT>(xv[s], upper, op[s]);
        load_x(nxt);
        __builtin_amdgcn_sched_barrier(kPinLoads);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < NMAT; ++q) {
                u32x4_t w = wv[t][q];
                load_w(t, q, nxt);
                __builtin_amdgcn_sched_barrier(kPinLoads);
                G::exchange(w);
                // the group's scales of this lane's row: 4 (Q4) or 2 (Q8_0)
                // consecutive entries
                const uint16_t* sr = sst + (q * ROWS + t * 16 + ln) * srl + grp * BPG;
                uint32_t sc[2];
                if constexpr (BPG == 4) {
                    const uint2 v = *reinterpret_cast<const uint2*>(sr);
                    sc[0] = v.x;
                    sc[1] = v.y;
                } else {
                    sc[0] = *reinterpret_cast<const uint32_t*>(sr);
                    sc[1] = sc[0];
                }
#pragma unroll
                for (int s = 0; s < BPG; ++s) {
                    // a block past K has a zero scale in LDS and adds exactly zero
                    const float d = f16_bits_to_f32(static_cast<uint16_t>(sc[s >> 1] >> (16 * (s & 1))));
                    const f32x4_t dot = block_dot<MT>(op[s], G::codes(w, s));
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[t][q][i] = __builtin_fmaf(d, dot[i], acc[t][q][i]);
                }
            }
    }

    // panels of at most 8 rows: rows 8-15 of D hold the middle parts of rows 0-7
    if constexpr (MT <= 8) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[t][q][i] = swap32_add(acc[t][q][i], acc[t][q][i]);
    }
    // the partial sums take the place of the scale rows
    float* const red = reinterpret_cast<float*>(lds);
    __syncthreads();
    if (MT > 8 || lane < 32) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[(((wave * NT + t) * NMAT + q) * MTO + 4 * lg + i) * 16 + ln] = acc[t][q][i];
    }
    __syncthreads();

    // outputs: partial sums added in wave order
    for (int idx = threadIdx.x; idx < NT * MTO * 16; idx += NW * 64) {
        const int t = idx / (MTO * 16), m = (idx / 16) % MTO, n = idx % 16;
        float v[NMAT];
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            float s = 0.f;
            for (int w = 0; w < NW; ++w) s += red[(((w * NT + t) * NMAT + q) * MTO + m) * 16 + n];
            v[q] = s * G::kOutScale;
        }
        const int row = (tb + t) * 16 + n;
        if (tb + t < te && m < M && row < N)
            y[static_cast<size_t>(m) * N + row] = MODE == Mode::SwiGLU ? swiglu_f32(v[0], v[NMAT - 1]) : v[0];
    }
}

constexpr int kMfmaWaves = static_cast<int>(plan::kMfmaWaves);
constexpr int kLdsLimit = static_cast<int>(plan::kLdsBytes);

template <Fmt F, Mode MODE, int MT, int NT>
hipError_t launch_nt(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                     const float* x, float* y, int M, int N, int K, hipStream_t stream) {
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    const int ntiles = (N + 15) / 16;
    // one workgroup per CU while that keeps NT tiles or fewer per workgroup
    const int grid = max(min(ntiles, device_cus()), (ntiles + NT - 1) / NT);
    const int lds = static_cast<int>(plan::mfma_lds_bytes(kMfmaWaves, NT, NMAT, MT <= 8 ? 8 : 16, K / kBlock));
    if (lds > kLdsLimit) return hipErrorInvalidValue;
    hipLaunchKernelGGL((qmv_f32_mfma<F, MODE, MT, NT, kMfmaWaves>), dim3(grid), dim3(kMfmaWaves * 64), lds, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb, x, y, M, N, K);
    return hipGetLastError();
}

template <Fmt F, Mode MODE, int MT>
hipError_t launch_mt(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                     const float* x, float* y, int M, int N, int K, hipStream_t stream) {
    switch (plan::mfma_nt(M, N, device_cus())) {
        case 1: return launch_nt<F, MODE, MT, 1>(wa, sa, wb, sb, x, y, M, N, K, stream);
        case 2: return launch_nt<F, MODE, MT, 2>(wa, sa, wb, sb, x, y, M, N, K, stream);
        case 3: return launch_nt<F, MODE, MT, 3>(wa, sa, wb, sb, x, y, M, N, K, stream);
        case 4: return launch_nt<F, MODE, MT, 4>(wa, sa, wb, sb, x, y, M, N, K, stream);
        case 5: return launch_nt<F, MODE, MT, 5>(wa, sa, wb, sb, x, y, M, N, K, stream);
        default: break;
    }
    // six tiles per workgroup only for panels of up to 8 rows (plan::mfma_max_nt)
    if constexpr (MT <= 8) return launch_nt<F, MODE, MT, 6>(wa, sa, wb, sb, x, y, M, N, K, stream);
    return hipErrorInvalidValue;
}

template <Fmt F, Mode MODE>
hipError_t launch_fm(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                     const float* x, float* y, int M, int N, int K, hipStream_t stream) {
    if (M <= 8) return launch_mt<F, MODE, 8>(wa, sa, wb, sb, x, y, M, N, K, stream);
    return launch_mt<F, MODE, 16>(wa, sa, wb, sb, x, y, M, N, K, stream);
}

}  // namespace

hipError_t launch_qmv_f32_mfma(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa,
                               const void* wb, const uint16_t* sb, const float* x, float* y,
                               int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (!plan::mfma_supported(fmt, M, N, K, device_cus())) return hipErrorInvalidValue;
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (fmt == Fmt::Q4 && mode == Mode::Plain) return launch_fm<Fmt::Q4, Mode::Plain>(wa, sa, wb, sb, x, y, m, n, k, stream);
    if (fmt == Fmt::Q4 && mode == Mode::SwiGLU) return launch_fm<Fmt::Q4, Mode::SwiGLU>(wa, sa, wb, sb, x, y, m, n, k, stream);
    if (fmt == Fmt::Q8_0 && mode == Mode::Plain) return launch_fm<Fmt::Q8_0, Mode::Plain>(wa, sa, wb, sb, x, y, m, n, k, stream);
    if (fmt == Fmt::Q8_0 && mode == Mode::SwiGLU) return launch_fm<Fmt::Q8_0, Mode::SwiGLU>(wa, sa, wb, sb, x, y, m, n, k, stream);
    return hipErrorInvalidValue;
}

}  // namespace qbd
