// Block-quantized weights x Q8 activations on gfx950: exact int32 block
// dots with v_dot4_i32_i8, then the fp32 scaled sum over blocks.
//
// The Q8 x Q8 fused matmul (Lumen v0.4.0 release page, "Phase 7.M - Q8xQ8
// AVX2 int dot": an exact integer block dot; "Phase 7.O - 4-accumulator VNNI
// kernel": one fp32 sub-accumulation per block) and its 4-bit-weight form
// for the gate/up consumer (LSE v0.4.16 release page, "Combined M8 Q4
// gate/up execution").
//
// y[m,n] = sum_b (d_w[n,b] * d_x[m,b]) * dot[m,n,b]; each block dot is
// formed whole, in int32, before it is scaled.  Q8_0 lanes own 16 codes
// (half a block) and add the partner lane's half with one DPP step; Q4
// lanes own a whole block (16 bytes).  4-bit codes become q - 8 as int8
// with the byte-parallel (q + 0x78) ^ 0x80.
#include "device_common.hpp"
#include "launch.hpp"

namespace qbd {
namespace {

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// 4 nibbles (low or high halves of 4 bytes) as 4 signed int8 values q - 8.
__device__ __forceinline__ uint32_t q4_lo_s8(uint32_t w) { return ((w & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u; }
__device__ __forceinline__ uint32_t q4_hi_s8(uint32_t w) { return (((w >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u; }

template <Fmt F> struct QChunk;

// Q8_0: chunk c = codes [16c, 16c+16); the block dot of block c/2 is the
// sum of chunks 2b and 2b+1, held by lanes 2i and 2i+1 of one sweep.
template <> struct QChunk<Fmt::Q8_0> {
    static constexpr int kCodes = 16;
    static constexpr int kActBytes = 16;
    __device__ static int block_of(int c) { return c >> 1; }
    __device__ static int dot(const uint4 w, const uint4* xa) {
        const uint4 a = xa[0];
        int s = sdot4(w.x, a.x, 0);
        s = sdot4(w.y, a.y, s);
        s = sdot4(w.z, a.z, s);
        s = sdot4(w.w, a.w, s);
        return s;
    }
    // full block dot in the even lane of each pair (odd lanes return 0)
    __device__ static int finish(int half, int lane) {
        const int other = __builtin_amdgcn_update_dpp(0, half, 0xB1, 0xF, 0xF, false);  // lane ^ 1
        return (lane & 1) ? 0 : half + other;
    }
    __device__ static bool owns_block(int lane) { return (lane & 1) == 0; }
    // a weight chunk ready for several activation rows (nothing to unpack)
    struct Prep {
        uint4 w;
    };
    __device__ static Prep prep(const uint4 w) { return {w}; }
    __device__ static int dot_prep(const Prep& p, const uint4* xa) { return dot(p.w, xa); }
};

// Q4: chunk c = block c, 16 bytes of nibbles against 32 activation codes.
template <> struct QChunk<Fmt::Q4> {
    static constexpr int kCodes = 32;
    static constexpr int kActBytes = 32;
    __device__ static int block_of(int c) { return c; }
    __device__ static int dot(const uint4 w, const uint4* xa) {
        const uint4 a0 = xa[0], a1 = xa[1];  // codes 0..15, 16..31
        int s = sdot4(q4_lo_s8(w.x), a0.x, 0);
        s = sdot4(q4_lo_s8(w.y), a0.y, s);
        s = sdot4(q4_lo_s8(w.z), a0.z, s);
        s = sdot4(q4_lo_s8(w.w), a0.w, s);
        s = sdot4(q4_hi_s8(w.x), a1.x, s);
        s = sdot4(q4_hi_s8(w.y), a1.y, s);
        s = sdot4(q4_hi_s8(w.z), a1.z, s);
        s = sdot4(q4_hi_s8(w.w), a1.w, s);
        return s;
    }
    __device__ static int finish(int full, int) { return full; }
    __device__ static bool owns_block(int) { return true; }
    // a weight chunk unpacked once for several activation rows: the same
    // signed bytes q - 8 and the same dot4 chain as dot()
    struct Prep {
        uint32_t lo[4], hi[4];
    };
    __device__ static Prep prep(const uint4 w) {
        return {{q4_lo_s8(w.x), q4_lo_s8(w.y), q4_lo_s8(w.z), q4_lo_s8(w.w)},
                {q4_hi_s8(w.x), q4_hi_s8(w.y), q4_hi_s8(w.z), q4_hi_s8(w.w)}};
    }
    __device__ static int dot_prep(const Prep& p, const uint4* xa) {
        const uint4 a0 = xa[0], a1 = xa[1];
        int s = sdot4(p.lo[0], a0.x, 0);
        s = sdot4(p.lo[1], a0.y, s);
        s = sdot4(p.lo[2], a0.z, s);
        s = sdot4(p.lo[3], a0.w, s);
        s = sdot4(p.hi[0], a1.x, s);
        s = sdot4(p.hi[1], a1.y, s);
        s = sdot4(p.hi[2], a1.z, s);
        s = sdot4(p.hi[3], a1.w, s);
        return s;
    }
    // The same block dot from the unbiased nibbles, for a staged panel whose
    // chunk sums are known: sum (q - 8) x = sum_lo q x + (sum_hi 8q x) / 8 -
    // 8 sum x, with the low nibbles as bytes q (one AND per 4 codes), the
    // high ones as bytes 8q (a shift and an AND; 8q <= 120 stays a positive
    // signed byte) and nsx8 = -8 sum x of the chunk.  Every step is exact
    // integer arithmetic, so the result equals dot() bit for bit, in fewer
    // VALU operations.
    __device__ static int dot_staged(const uint4 w, const uint4* xa, int nsx8) {
        const uint4 a0 = xa[0], a1 = xa[1];
        constexpr uint32_t kLo = 0x0F0F0F0Fu, kHi8 = 0x78787878u;
        int lo = sdot4(w.x & kLo, a0.x, 0);
        lo = sdot4(w.y & kLo, a0.y, lo);
        lo = sdot4(w.z & kLo, a0.z, lo);
        lo = sdot4(w.w & kLo, a0.w, lo);
        int hi = sdot4((w.x >> 1) & kHi8, a1.x, 0);
        hi = sdot4((w.y >> 1) & kHi8, a1.y, hi);
        hi = sdot4((w.z >> 1) & kHi8, a1.z, hi);
        hi = sdot4((w.w >> 1) & kHi8, a1.w, hi);
        return lo + (hi >> 3) + nsx8;  // hi is a multiple of 8: the shift is exact
    }
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Weight chunks are read once per call: stream them with a non-temporal load.
__device__ __forceinline__ uint4 load_stream(const uint8_t* __restrict__ p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <Fmt F>
__device__ __forceinline__ size_t qrow_bytes(int K) {
    return F == Fmt::Q8_0 ? static_cast<size_t>(K) : static_cast<size_t>(K) / 2;
}

// One output row per wave, MT activation rows per pass.
template <Fmt F, Mode MODE, int MT>
__global__ __launch_bounds__(256) void qmm_q8act_generic(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, float* __restrict__ y,
    int M, int N, int K) {
    using C = QChunk<F>;
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    // sweeps cover whole chunks; lanes past the end hold zero dots
    const int nsweeps = (nchunks + kWave - 1) / kWave;
    const uint8_t* ra = wa + static_cast<size_t>(n) * qrow_bytes<F>(K);
    const uint16_t* rsa = sa + static_cast<size_t>(n) * nblocks;
    const uint8_t* rb = MODE == Mode::SwiGLU ? wb + static_cast<size_t>(n) * qrow_bytes<F>(K) : nullptr;
    const uint16_t* rsb = MODE == Mode::SwiGLU ? sb + static_cast<size_t>(n) * nblocks : nullptr;

    for (int m0 = blockIdx.y * MT; m0 < M; m0 += gridDim.y * MT) {
        float acc_a[MT], acc_b[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) { acc_a[i] = 0.f; acc_b[i] = 0.f; }
        for (int s = 0; s < nsweeps; ++s) {
            const int c = s * kWave + lane;
            const bool live = c < nchunks;
            uint4 w = make_uint4(0, 0, 0, 0), w2 = make_uint4(0, 0, 0, 0);
            float dw = 0.f, dw2 = 0.f;
            if (live) {
                w = *reinterpret_cast<const uint4*>(ra + static_cast<size_t>(c) * 16);
                dw = f16_bits_to_f32(rsa[C::block_of(c)]);
                if constexpr (MODE == Mode::SwiGLU) {
                    w2 = *reinterpret_cast<const uint4*>(rb + static_cast<size_t>(c) * 16);
                    dw2 = f16_bits_to_f32(rsb[C::block_of(c)]);
                }
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if (m0 + i < M) {  // wave-uniform
                    const size_t row = static_cast<size_t>(m0 + i);
                    uint4 xa[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
                    float dx = 0.f;
                    if (live) {
                        const uint4* p = reinterpret_cast<const uint4*>(
                            xq + row * K + static_cast<size_t>(c) * C::kCodes);
                        xa[0] = p[0];
                        if constexpr (C::kActBytes == 32) xa[1] = p[1];
                        dx = xd[row * nblocks + C::block_of(c)];
                    }
                    const int dot = C::finish(C::dot(w, xa), lane);
                    if (live && C::owns_block(lane))
                        acc_a[i] = __builtin_fmaf(dw * dx, static_cast<float>(dot), acc_a[i]);
                    if constexpr (MODE == Mode::SwiGLU) {
                        const int dot2 = C::finish(C::dot(w2, xa), lane);
                        if (live && C::owns_block(lane))
                            acc_b[i] = __builtin_fmaf(dw2 * dx, static_cast<float>(dot2), acc_b[i]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            float va[1] = {acc_a[i]};
            wave_reduce<1>(va);
            float out = va[0];
            if constexpr (MODE == Mode::SwiGLU) {
                float vb[1] = {acc_b[i]};
                wave_reduce<1>(vb);
                out = swiglu_f32(va[0], vb[0]);
            }
            if (lane == 0 && m0 + i < M) y[static_cast<size_t>(m0 + i) * N + n] = out;
        }
    }
}

template <Fmt F, Mode MODE, int MT>
hipError_t launch_generic(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                          const int8_t* xq, const float* xd, float* y, int M, int N, int K,
                          hipStream_t stream) {
    const int gx = (N + 3) / 4;
    const int chunks = (M + MT - 1) / MT;
    const int gy = chunks < 65535 ? chunks : 65535;
    hipLaunchKernelGGL((qmm_q8act_generic<F, MODE, MT>), dim3(gx, gy), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                       xq, xd, y, M, N, K);
    return hipGetLastError();
}

// M = 1, quantizing x inside the product, for short rows and few enough
// of them that the repeated quantization stays small: every workgroup
// quantizes the whole fp32 x into LDS with the functions of the
// quantization kernel (so its codes and scales are bit for bit those of
// quantize_act_q8_0), then each of its four waves forms one output row with
// the per-row kernel's sums in the per-row kernel's order (which is also
// the staged kernel's: chunk j * 64 + lane, sweeps in order, the same DPP
// tree), so y is bit for bit that of quantize_act_q8_0 followed by the
// product.  The row's NS
// weight sweeps are loaded first (clamped, unconditional), so they are in
// flight while x is read and quantized; workgroup 0 also writes the codes
// and scales out.
template <Fmt F, Mode MODE, int NS>
__global__ __launch_bounds__(256) void qmm_q8act_m1_qx(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, int8_t* __restrict__ xq_out, float* __restrict__ xd_out,
    float* __restrict__ y, int N, int K) {
    using C = QChunk<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int KMAX = NS * kWave * C::kCodes;  // codes the sweeps cover
    constexpr int R = (KMAX / 8 + 255) / 256;     // quantization rounds of 256 groups of 8
    __shared__ __align__(16) int8_t xs[KMAX];
    __shared__ float dxs[KMAX / kBlock];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = blockIdx.x * 4 + wave;
    const size_t n = static_cast<size_t>(min(row, N - 1));  // a wave past N computes row N - 1, stores nothing
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    const size_t rbytes = qrow_bytes<F>(K);
    const uint8_t* const wm[2] = {wa, wb};
    const uint16_t* const sm[2] = {sa, sb};

    uint4 w[NMAT][NS];
    uint16_t ws[NMAT][NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c = min(s * kWave + lane, nchunks - 1);
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            w[q][s] = load_stream(wm[q] + n * rbytes + static_cast<size_t>(c) * 16);
            ws[q][s] = sm[q][n * nblocks + C::block_of(c)];
        }
    }

    // quantize x: group g = 8 consecutive values, groups 4b .. 4b + 3 form
    // block b and sit in one lane quad, so the block maximum is two DPP steps
    const int ngroups = K / 8;
    float4 va[R], vb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const size_t gc = static_cast<size_t>(min(r * 256 + tid, ngroups - 1));
        va[r] = *reinterpret_cast<const float4*>(x + 8 * gc);
        vb[r] = *reinterpret_cast<const float4*>(x + 8 * gc + 4);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r * 256 >= ngroups) break;  // workgroup-uniform
        const int gi = r * 256 + tid;
        const bool live = gi < ngroups;
        float v[8] = {va[r].x, va[r].y, va[r].z, va[r].w, vb[r].x, vb[r].y, vb[r].z, vb[r].w};
        if (!live) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = fmaxf(amax, dpp_shuffle<0xB1>(amax));
        amax = fmaxf(amax, dpp_shuffle<0x4E>(amax));
        const float d = q8_block_scale(amax);
        if (live) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo |= static_cast<uint32_t>(static_cast<uint8_t>(q8_quantize_one(v[i], d))) << (8 * i);
                hi |= static_cast<uint32_t>(static_cast<uint8_t>(q8_quantize_one(v[4 + i], d))) << (8 * i);
            }
            *reinterpret_cast<uint2*>(xs + 8 * gi) = make_uint2(lo, hi);
            if ((gi & 3) == 0) dxs[gi >> 2] = d;
            if (blockIdx.x == 0) {
                *reinterpret_cast<uint2*>(xq_out + 8 * gi) = make_uint2(lo, hi);
                if ((gi & 3) == 0) xd_out[gi >> 2] = d;
            }
        }
    }
    __syncthreads();

    float acc[NMAT];
#pragma unroll
    for (int q = 0; q < NMAT; ++q) acc[q] = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c = s * kWave + lane;
        const bool live = c < nchunks;
        // chunks past K read codes and scales past K's end in LDS (in
        // bounds, never added)
        uint4 xa[2];
        xa[0] = *reinterpret_cast<const uint4*>(xs + static_cast<size_t>(c) * C::kCodes);
        if constexpr (C::kActBytes == 32) xa[1] = *reinterpret_cast<const uint4*>(xs + static_cast<size_t>(c) * C::kCodes + 16);
        const float dx = dxs[C::block_of(c)];
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            const int dot = C::finish(C::dot(w[q][s], xa), lane);
            if (live && C::owns_block(lane))
                acc[q] = __builtin_fmaf(f16_bits_to_f32(ws[q][s]) * dx, static_cast<float>(dot), acc[q]);
        }
    }
    float va0[1] = {acc[0]};
    wave_reduce<1>(va0);
    float out = va0[0];
    if constexpr (MODE == Mode::SwiGLU) {
        float vb0[1] = {acc[NMAT - 1]};
        wave_reduce<1>(vb0);
        out = swiglu_f32(va0[0], vb0[0]);
    }
    if (lane == 0 && row < N) y[n] = out;
}

template <Fmt F, Mode MODE>
hipError_t launch_m1_qx(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb, const float* x,
                        int8_t* xq, float* xd, float* y, int N, int K, hipStream_t stream) {
    const int gx = (N + 3) / 4;
    const int ns = static_cast<int>(plan::m1_sweeps(F, K));
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(gx), dim3(256), 0, stream, static_cast<const uint8_t*>(wa), sa,
                           static_cast<const uint8_t*>(wb), sb, x, xq, xd, y, N, K);
        return hipGetLastError();
    };
    switch (ns) {
        case 1: return go(qmm_q8act_m1_qx<F, MODE, 1>);
        case 2: return go(qmm_q8act_m1_qx<F, MODE, 2>);
        case 3: return go(qmm_q8act_m1_qx<F, MODE, 3>);
        case 4: return go(qmm_q8act_m1_qx<F, MODE, 4>);
        default: break;
    }
    if constexpr (F == Fmt::Q8_0) {
        switch (ns) {
            case 5: return go(qmm_q8act_m1_qx<F, MODE, 5>);
            case 6: return go(qmm_q8act_m1_qx<F, MODE, 6>);
            case 7: return go(qmm_q8act_m1_qx<F, MODE, 7>);
            case 8: return go(qmm_q8act_m1_qx<F, MODE, 8>);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

// M = 1 with the activation panel staged once per workgroup (one per CU).
// Codes and scales of x sit in LDS part-major, so lane l of sweep j reads
// the 16-byte parts of chunk j * 64 + l with consecutive lanes on
// consecutive addresses; a chunk past K meets zero codes and a zero scale.
// A workgroup of NW waves owns a contiguous range of rows, wave w takes rows
// row_begin + w + NW g (NW chosen per shape so that the rows spread evenly).
// An item is a row and a group of S consecutive sweeps, whose S weight
// chunks per lane are loaded at once (non-temporal: each weight is read
// once); two register sets A and B hold alternate items, so the next item's
// loads are in flight while the current one is multiplied.  Sweeps past the
// row's last (when S does not divide the sweep count) load a clamped chunk
// and meet zero activations, adding exactly zero.  Per row: one exact int32
// block dot per chunk (Q8_0: two lanes' halves added by one DPP step),
// scaled by d_w d_x into the lane's fp32 accumulator, sweeps in order, then
// the fixed DPP / permlane tree.  The grouping and NW leave that order
// unchanged, and the plain and the SwiGLU kernels share it, so fused ==
// unfused holds bitwise.  Loads are unconditional (clamped rows and chunks)
// and outputs are gathered in LDS.
//
// QX: the workgroup quantizes the fp32 panel itself while staging it, with
// the rule of quantize_act_q8_0 (q8_block_scale, q8_quantize_one: four
// lanes per block, the block maximum by two DPP steps), so the staged codes
// and scales, and hence every output, are those of quantize_act_q8_0
// followed by the product; workgroup 0 also writes the quantized panel out.
// A separate producer launch costs more than re-quantizing K values in
// every workgroup.
struct ActIn {
    const int8_t* xq;  // staged codes and scales (QX = false)
    const float* xd;
    const float* x;    // fp32 panel to quantize (QX = true)
    int8_t* xq_out;    // where workgroup 0 writes the quantized panel (QX = true)
    float* xd_out;
};

template <Fmt F, Mode MODE, int S, int NW, bool QX>
__global__ __launch_bounds__(NW * 64) void qmm_q8act_m1_staged(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const ActIn act, float* __restrict__ y, int N, int K, int J, int rows_per_wg) {
    using C = QChunk<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int AP = C::kActBytes / 16;  // 16-byte parts of a chunk's activation codes
    constexpr int NT = NW * 64;
    const int G = (J + S - 1) / S;         // sweep groups per row
    extern __shared__ __align__(16) uint4 lds_q[];
    uint4* xs = lds_q;                                                                       // [G*S][AP][64]
    float* dxs = reinterpret_cast<float*>(lds_q + static_cast<size_t>(G) * S * AP * kWave);  // [G*S][64]
    // 4-bit weights: -8 x (sum of the chunk's activation codes), per chunk
    int* nsx = reinterpret_cast<int*>(dxs + static_cast<size_t>(G) * S * kWave);             // [G*S][64] (Q4)
    float* yout = reinterpret_cast<float*>(nsx + (F == Fmt::Q4 ? static_cast<size_t>(G) * S * kWave : 0));  // [rows]
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    const size_t rbytes = qrow_bytes<F>(K);

    const int row_begin = blockIdx.x * rows_per_wg;
    const int row_end = min(row_begin + rows_per_wg, N);
    const int my_rows = row_end - row_begin > wave ? (row_end - row_begin - wave + NW - 1) / NW : 0;
    const int items = my_rows * G;

    struct Slot {
        uint4 w[NMAT][S];
        uint16_t s[NMAT][S];
    };
    int ig = 0, ir = 0;  // sweep group and row of the next item to load
    auto issue = [&](Slot& T) {
        const size_t row = static_cast<size_t>(min(row_begin + wave + NW * ir, row_end - 1));
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int c = min((ig * S + u) * kWave + lane, nchunks - 1);
            T.w[0][u] = load_stream(wa + row * rbytes + static_cast<size_t>(c) * 16);
            T.s[0][u] = sa[row * nblocks + C::block_of(c)];
            if constexpr (NMAT == 2) {
                T.w[1][u] = load_stream(wb + row * rbytes + static_cast<size_t>(c) * 16);
                T.s[1][u] = sb[row * nblocks + C::block_of(c)];
            }
        }
        if (++ig == G) { ig = 0; ++ir; }
    };
    // the first item's weights fly while the panel is staged
    Slot A, B;
    issue(A);

    if constexpr (QX) {
        // group g = 8 consecutive values, groups 4b .. 4b + 3 form block b
        // and sit in one lane quad (NT is a multiple of 64); every lane runs
        // every round, so the DPP steps see whole quads
        const int ngroups = K / 8;
        uint8_t* const xsb = reinterpret_cast<uint8_t*>(xs);
        // R rounds per batch: their loads (clamped to the last group, so
        // unconditional) are issued together, one memory round trip per batch
        constexpr int R = plan::kQ8M1QuantRounds;
        for (int g0 = 0; g0 < ngroups; g0 += R * NT) {
            const int nr = min(R, (ngroups - g0 + NT - 1) / NT);  // live rounds of this batch
            float4 va[R], vb[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r < nr) {  // wave-uniform
                    const size_t gc = static_cast<size_t>(min(g0 + r * NT + tid, ngroups - 1));
                    va[r] = *reinterpret_cast<const float4*>(act.x + 8 * gc);
                    vb[r] = *reinterpret_cast<const float4*>(act.x + 8 * gc + 4);
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r >= nr) break;  // wave-uniform
                const int gi = g0 + r * NT + tid;
                const bool live = gi < ngroups;
                float v[8] = {va[r].x, va[r].y, va[r].z, va[r].w, vb[r].x, vb[r].y, vb[r].z, vb[r].w};
                if (!live) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = 0.f;
                }
                float amax = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
                amax = fmaxf(amax, dpp_shuffle<0xB1>(amax));
                amax = fmaxf(amax, dpp_shuffle<0x4E>(amax));
                const float d = q8_block_scale(amax);
                if (live) {
                    uint32_t lo = 0, hi = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        lo |= static_cast<uint32_t>(static_cast<uint8_t>(q8_quantize_one(v[i], d))) << (8 * i);
                        hi |= static_cast<uint32_t>(static_cast<uint8_t>(q8_quantize_one(v[4 + i], d))) << (8 * i);
                    }
                    // codes 8 gi .. 8 gi + 7: half of one 16-byte part of chunk c
                    const int code0 = 8 * gi;
                    const int c = code0 / C::kCodes, o = code0 % C::kCodes;
                    const int j = c / kWave, l = c % kWave, p = o / 16, half = (o / 8) & 1;
                    *reinterpret_cast<uint2*>(xsb + ((static_cast<size_t>(j) * AP + p) * kWave + l) * 16 + 8 * half) =
                        make_uint2(lo, hi);
                    const int blk = gi >> 2;
                    if ((gi & 3) == 0) {
                        if constexpr (F == Fmt::Q8_0) {
                            dxs[2 * blk] = d;
                            dxs[2 * blk + 1] = d;
                        } else {
                            dxs[blk] = d;
                        }
                    }
                    if (blockIdx.x == 0) {
                        *reinterpret_cast<uint2*>(act.xq_out + code0) = make_uint2(lo, hi);
                        if ((gi & 3) == 0) act.xd_out[blk] = d;
                    }
                }
            }
        }
        // chunks past K: zero codes and a zero scale
        for (int i = tid; i < G * S * AP * kWave; i += NT) {
            const int j = i / (AP * kWave), l = i % kWave;
            if (j * kWave + l >= nchunks) xs[i] = make_uint4(0, 0, 0, 0);
        }
        for (int c = nchunks + tid; c < G * S * kWave; c += NT) dxs[c] = 0.f;
    } else {
        for (int i = tid; i < G * S * AP * kWave; i += NT) {
            const int j = i / (AP * kWave), p = (i / kWave) % AP, l = i % kWave;
            const int c = j * kWave + l;
            xs[i] = c < nchunks
                        ? *reinterpret_cast<const uint4*>(act.xq + static_cast<size_t>(c) * C::kCodes + 16 * p)
                        : make_uint4(0, 0, 0, 0);
        }
        for (int c = tid; c < G * S * kWave; c += NT) dxs[c] = c < nchunks ? act.xd[C::block_of(c)] : 0.f;
    }
    __syncthreads();
    if constexpr (F == Fmt::Q4) {
        // the chunk sums of the staged codes (chunks past K hold zeros)
        for (int c = tid; c < G * S * kWave; c += NT) {
            const int j = c / kWave, l = c % kWave;
            const uint4 p0 = xs[(j * AP) * kWave + l], p1 = xs[(j * AP + 1) * kWave + l];
            constexpr uint32_t kOnes = 0x01010101u;
            int sum = sdot4(p0.x, kOnes, 0);
            sum = sdot4(p0.y, kOnes, sum);
            sum = sdot4(p0.z, kOnes, sum);
            sum = sdot4(p0.w, kOnes, sum);
            sum = sdot4(p1.x, kOnes, sum);
            sum = sdot4(p1.y, kOnes, sum);
            sum = sdot4(p1.z, kOnes, sum);
            sum = sdot4(p1.w, kOnes, sum);
            nsx[c] = -8 * sum;
        }
        __syncthreads();
    }

    float acc[NMAT];
    int g = 0, rr = 0;  // sweep group and row of the item being multiplied
    auto compute = [&](const Slot& T) {
        if (g == 0) {
#pragma unroll
            for (int q = 0; q < NMAT; ++q) acc[q] = 0.f;
        }
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int j = g * S + u;
            uint4 xa[2];
#pragma unroll
            for (int p = 0; p < AP; ++p) xa[p] = xs[(j * AP + p) * kWave + lane];
            const float dx = dxs[j * kWave + lane];
            int nsx8 = 0;
            if constexpr (F == Fmt::Q4) nsx8 = nsx[j * kWave + lane];
#pragma unroll
            for (int q = 0; q < NMAT; ++q) {
                int dot;  // block dot (0 in odd Q8_0 lanes)
                if constexpr (F == Fmt::Q4) {
                    dot = C::dot_staged(T.w[q][u], xa, nsx8);
                } else {
                    dot = C::finish(C::dot(T.w[q][u], xa), lane);
                }
                acc[q] = __builtin_fmaf(static_cast<float>(dot), f16_bits_to_f32(T.s[q][u]) * dx, acc[q]);
            }
        }
        if (g == G - 1) {
            float va[1] = {acc[0]};
            wave_reduce<1>(va);
            float out = va[0];
            if constexpr (NMAT == 2) {
                float vb[1] = {acc[1]};
                wave_reduce<1>(vb);
                out = swiglu_f32(va[0], vb[0]);
            }
            if (lane == 0) yout[wave + NW * rr] = out;
        }
        if (++g == G) { g = 0; ++rr; }
    };

    for (int t = 0; t < items; t += 2) {
        issue(B);  // item t + 1 (past the last item: a clamped row, never used)
        compute(A);
        issue(A);  // item t + 2
        if (t + 1 < items) compute(B);
    }

    __syncthreads();
    for (int i = tid; i < row_end - row_begin; i += NT) y[row_begin + i] = yout[i];
}

template <Fmt F, Mode MODE, bool QX, int S, int NW>
hipError_t launch_m1_staged_nw(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                               const ActIn& act, float* y, int N, int K, hipStream_t stream) {
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    const int J = static_cast<int>(plan::m1_sweeps(F, K));
    const int rows_per_wg = static_cast<int>(plan::resident_rows(N, device_cus()));
    const int gx = (N + rows_per_wg - 1) / rows_per_wg;
    const size_t lds = static_cast<size_t>(plan::q8act_m1_lds_bytes(F, K, rows_per_wg, NMAT));
    if (lds > static_cast<size_t>(plan::kLdsBytes)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((qmm_q8act_m1_staged<F, MODE, S, NW, QX>), dim3(gx), dim3(NW * 64), lds, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb, act, y, N, K,
                       J, rows_per_wg);
    return hipGetLastError();
}

template <Fmt F, Mode MODE, bool QX, int S>
hipError_t launch_m1_staged_s(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                              const ActIn& act, float* y, int N, int K, hipStream_t stream) {
    switch (plan::q8act_m1_waves(N, device_cus())) {
        case 4: return launch_m1_staged_nw<F, MODE, QX, S, 4>(wa, sa, wb, sb, act, y, N, K, stream);
        case 8: return launch_m1_staged_nw<F, MODE, QX, S, 8>(wa, sa, wb, sb, act, y, N, K, stream);
        case 16: return launch_m1_staged_nw<F, MODE, QX, S, 16>(wa, sa, wb, sb, act, y, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

template <Fmt F, Mode MODE, bool QX>
hipError_t launch_m1_staged(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                            const ActIn& act, float* y, int N, int K, hipStream_t stream) {
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    switch (plan::q8act_m1_group(F, K, NMAT)) {
        case 1: return launch_m1_staged_s<F, MODE, QX, 1>(wa, sa, wb, sb, act, y, N, K, stream);
        case 2: return launch_m1_staged_s<F, MODE, QX, 2>(wa, sa, wb, sb, act, y, N, K, stream);
        case 3: return launch_m1_staged_s<F, MODE, QX, 3>(wa, sa, wb, sb, act, y, N, K, stream);
        case 4: return launch_m1_staged_s<F, MODE, QX, 4>(wa, sa, wb, sb, act, y, N, K, stream);
        case 5: return launch_m1_staged_s<F, MODE, QX, 5>(wa, sa, wb, sb, act, y, N, K, stream);
        default: break;
    }
    if constexpr (NMAT == 1) {
        switch (plan::q8act_m1_group(F, K, NMAT)) {
            case 6: return launch_m1_staged_s<F, MODE, QX, 6>(wa, sa, wb, sb, act, y, N, K, stream);
            case 7: return launch_m1_staged_s<F, MODE, QX, 7>(wa, sa, wb, sb, act, y, N, K, stream);
            case 8: return launch_m1_staged_s<F, MODE, QX, 8>(wa, sa, wb, sb, act, y, N, K, stream);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

template <bool QX>
hipError_t launch_m1_staged_any(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa, const void* wb,
                                const uint16_t* sb, const ActIn& act, float* y, int N, int K, hipStream_t stream) {
    if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
        return launch_m1_staged<Fmt::Q8_0, Mode::Plain, QX>(wa, sa, wb, sb, act, y, N, K, stream);
    if (fmt == Fmt::Q4 && mode == Mode::Plain)
        return launch_m1_staged<Fmt::Q4, Mode::Plain, QX>(wa, sa, wb, sb, act, y, N, K, stream);
    if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
        return launch_m1_staged<Fmt::Q4, Mode::SwiGLU, QX>(wa, sa, wb, sb, act, y, N, K, stream);
    return hipErrorInvalidValue;
}

// 2 <= M <= 8 activation rows (MT: M padded to 2, 4 or 8) against
// long weight rows.  One workgroup of 16 waves owns up to 16 RW
// consecutive weight rows; wave w takes rows row_begin + w + 16 r (r < RW).
// The Q8 panel (all MT rows, SW sweeps of 64 chunks per step) is staged in
// LDS step by step, double-buffered: while step k is multiplied, the
// weights of steps k + 1 and k + 2 are in flight in two more register sets
// (a step's loads alone do not cover the memory latency) and step k + 1's
// panel is in registers on its way to the other LDS buffer.  The panel is read from
// L2 once per workgroup and each weight row once (the dot4 kernel reads the
// panel once per weight row).  Per lane, each (weight row, activation row)
// pair sums its chunks in sweep order as fma(dot, d_w d_x, acc), then the
// wave's DPP / permlane tree: the order of the dot4 kernel, so the outputs
// are bitwise equal to it.  Chunks past K and rows past M are staged as
// zero codes with a zero scale; weight loads are clamped in bounds.
template <Fmt F, Mode MODE, int MT, int SW, int RW>
__global__ __launch_bounds__(1024) void qmm_q8act_panel_staged(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const int8_t* __restrict__ xq, const float* __restrict__ xd, float* __restrict__ y,
    int M, int N, int K, int rows_per_wg) {
    using C = QChunk<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int AP = C::kActBytes / 16;
    constexpr int NW = 16, NT = NW * kWave;
    constexpr int kQuads = MT * SW * AP * kWave;     // code quads of one buffer
    constexpr int kScales = MT * SW * kWave;         // activation scales of one buffer
    constexpr int kBufQuads = kQuads + kScales / 4;  // one buffer in uint4 units
    constexpr int kQPT = (kQuads + NT - 1) / NT;     // staged quads per thread
    constexpr int kSPT = (kScales + NT - 1) / NT;
    extern __shared__ __align__(16) uint4 lds_p[];   // two buffers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunks = K / C::kCodes, nblocks = K / kBlock;
    const int nsweeps = (nchunks + kWave - 1) / kWave;
    const int nsteps = (nsweeps + SW - 1) / SW;
    const size_t rbytes = qrow_bytes<F>(K);
    const int row_begin = blockIdx.x * rows_per_wg;
    const int row_end = min(row_begin + rows_per_wg, N);
    // live rows of this wave (wave-uniform); rows past them are clamped copies
    const int nr = row_end - row_begin > wave ? (row_end - row_begin - wave + NW - 1) / NW : 0;
    size_t wrow[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) wrow[r] = static_cast<size_t>(min(row_begin + wave + NW * r, row_end - 1));

    // ---- the panel of step k: global -> registers -> LDS buffer
    uint4 pq[kQPT];
    float ps[kSPT];
    auto panel_load = [&](int k) {
#pragma unroll
        for (int t = 0; t < kQPT; ++t) {
            const int i = tid + t * NT;
            const int l = i % kWave, p = (i / kWave) % AP, u = (i / (kWave * AP)) % SW, m = i / (kWave * AP * SW);
            const int c = (k * SW + u) * kWave + l;
            const bool ok = i < kQuads && m < M && c < nchunks;
            const size_t mm = static_cast<size_t>(min(m, M - 1)), cc = static_cast<size_t>(min(c, nchunks - 1));
            const uint4 v = *reinterpret_cast<const uint4*>(xq + mm * K + cc * C::kCodes + 16 * p);
            pq[t] = ok ? v : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < kSPT; ++t) {
            const int i = tid + t * NT;
            const int l = i % kWave, u = (i / kWave) % SW, m = i / (kWave * SW);
            const int c = (k * SW + u) * kWave + l;
            const bool ok = i < kScales && m < M && c < nchunks;
            const size_t mm = static_cast<size_t>(min(m, M - 1));
            const float v = xd[mm * nblocks + C::block_of(min(c, nchunks - 1))];
            ps[t] = ok ? v : 0.f;
        }
    };
    auto panel_store = [&](int b) {
        uint4* q = lds_p + b * kBufQuads;
        float* sc = reinterpret_cast<float*>(q + kQuads);
#pragma unroll
        for (int t = 0; t < kQPT; ++t) {
            const int i = tid + t * NT;
            if (i < kQuads) q[i] = pq[t];
        }
#pragma unroll
        for (int t = 0; t < kSPT; ++t) {
            const int i = tid + t * NT;
            if (i < kScales) sc[i] = ps[t];
        }
    };

    // ---- the weights of step k for this wave's rows
    struct Wt {
        uint4 w[NMAT][RW][SW];
        uint16_t s[NMAT][RW][SW];
    };
    auto wload = [&](Wt& T, int k) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int u = 0; u < SW; ++u) {
                const int c = min((k * SW + u) * kWave + lane, nchunks - 1);
                T.w[0][r][u] = load_stream(wa + wrow[r] * rbytes + static_cast<size_t>(c) * 16);
                T.s[0][r][u] = sa[wrow[r] * nblocks + C::block_of(c)];
                if constexpr (NMAT == 2) {
                    T.w[1][r][u] = load_stream(wb + wrow[r] * rbytes + static_cast<size_t>(c) * 16);
                    T.s[1][r][u] = sb[wrow[r] * nblocks + C::block_of(c)];
                }
            }
    };

    float acc[NMAT][RW][MT];
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[q][r][m] = 0.f;
    auto compute = [&](const Wt& T, int b) {
        const uint4* q = lds_p + b * kBufQuads;
        const float* sc = reinterpret_cast<const float*>(q + kQuads);
#pragma unroll
        for (int u = 0; u < SW; ++u) {
            // each weight chunk unpacked once, for all MT activation rows
            typename C::Prep pw[NMAT][RW];
            float dw[NMAT][RW];
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    if (r < nr) {  // wave-uniform
                        pw[mat][r] = C::prep(T.w[mat][r][u]);
                        dw[mat][r] = f16_bits_to_f32(T.s[mat][r][u]);
                    }
                }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                uint4 xa[2];
#pragma unroll
                for (int p = 0; p < AP; ++p) xa[p] = q[((m * SW + u) * AP + p) * kWave + lane];
                const float dx = sc[(m * SW + u) * kWave + lane];
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    if (r < nr) {  // wave-uniform
#pragma unroll
                        for (int mat = 0; mat < NMAT; ++mat) {
                            const int dot = C::finish(C::dot_prep(pw[mat][r], xa), lane);
                            acc[mat][r][m] = __builtin_fmaf(static_cast<float>(dot), dw[mat][r] * dx, acc[mat][r][m]);
                        }
                    }
                }
            }
        }
    };

    // three register sets: step k's weights are loaded two steps ahead (the
    // panel one step ahead, into the other LDS buffer)
    Wt W0, W1, W2;
    // Loads are unconditional, from step indices clamped to the last step
    // (past it they repeat the last step's addresses and are not used): a
    // load under a branch makes the compiler wait for every load in flight
    // before the next use, which would undo the prefetch.
    const int last = nsteps - 1;
    auto step = [&](int k, const Wt& cur, Wt& ahead) {
        const int b = k & 1;
        // the panel first: storing it then waits for it alone, and the
        // weights of step k + 2 stay in flight (loads complete in order)
        panel_load(min(k + 1, last));
        wload(ahead, min(k + 2, last));
        compute(cur, b);
        panel_store(b ^ 1);
        __syncthreads();
    };
    panel_load(0);
    wload(W0, 0);
    wload(W1, min(1, last));
    panel_store(0);
    __syncthreads();
    for (int k = 0; k < nsteps; k += 3) {
        step(k, W0, W2);
        if (k + 1 >= nsteps) break;
        step(k + 1, W1, W0);
        if (k + 2 >= nsteps) break;
        step(k + 2, W2, W1);
    }

    // ---- per (row, activation row): the wave's tree, then the output
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        if (r >= nr) break;  // wave-uniform
        const int row = row_begin + wave + NW * r;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float va[1] = {acc[0][r][m]};
            wave_reduce<1>(va);
            float out = va[0];
            if constexpr (NMAT == 2) {
                float vb[1] = {acc[NMAT - 1][r][m]};
                wave_reduce<1>(vb);
                out = swiglu_f32(va[0], vb[0]);
            }
            if (lane == 0 && m < M) y[static_cast<size_t>(m) * N + row] = out;
        }
    }
}

template <Fmt F, Mode MODE, int MT>
hipError_t launch_panel_staged_mt(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                                  const int8_t* xq, const float* xd, float* y, int M, int N, int K,
                                  hipStream_t stream) {
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int SW = static_cast<int>(plan::q8act_panel_sweeps(F, MT, NMAT));
    constexpr int RW = static_cast<int>(plan::q8act_panel_rows_per_wave(NMAT));
    const int rows_per_wg = static_cast<int>(plan::q8act_panel_rows(N, NMAT, device_cus()));
    const int gx = (N + rows_per_wg - 1) / rows_per_wg;
    const size_t lds = static_cast<size_t>(plan::q8act_panel_lds_bytes(F, MT, NMAT));
    if (lds > static_cast<size_t>(plan::kLdsBytes)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((qmm_q8act_panel_staged<F, MODE, MT, SW, RW>), dim3(gx), dim3(1024), lds, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb, xq, xd, y, M, N, K,
                       rows_per_wg);
    return hipGetLastError();
}

template <Fmt F, Mode MODE>
hipError_t launch_panel_staged(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                               const int8_t* xq, const float* xd, float* y, int M, int N, int K,
                               hipStream_t stream) {
    switch (plan::q8act_panel_mt(M)) {
        case 2: return launch_panel_staged_mt<F, MODE, 2>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 4: return launch_panel_staged_mt<F, MODE, 4>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        case 8: return launch_panel_staged_mt<F, MODE, 8>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
        default: return hipErrorInvalidValue;
    }
}

template <Fmt F, Mode MODE>
hipError_t dispatch(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                    const int8_t* xq, const float* xd, float* y, int M, int N, int K, int mt,
                    hipStream_t stream) {
    if (mt == 1) return launch_generic<F, MODE, 1>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
    if (mt == 2) return launch_generic<F, MODE, 2>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
    return launch_generic<F, MODE, 4>(wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
}

}  // namespace

hipError_t launch_qmm_q8act(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa,
                            const void* wb, const uint16_t* sb, const int8_t* xq,
                            const float* xd, float* y, int64_t M, int64_t N, int64_t K,
                            hipStream_t stream) {
    // Panels of 16 rows or more go to the matrix cores; fewer rows stay on
    // the VALU dot4 kernel (a 32-row MFMA tile would be mostly padding).
    const plan::Q8Plan p = plan::q8act_plan(fmt, M, N, K, device_cus());
    if (p.kernel == plan::Q8Kernel::Tile16Persist)
        return launch_qmm_q8_tile16_persist(fmt, mode, wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
    if (p.kernel == plan::Q8Kernel::Tile16)
        return launch_qmm_q8_tile16(fmt, mode, wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (p.kernel == plan::Q8Kernel::M1Staged)
        return launch_m1_staged_any<false>(fmt, mode, wa, sa, wb, sb, ActIn{xq, xd, nullptr, nullptr, nullptr}, y,
                                           n, k, stream);
    if (p.kernel == plan::Q8Kernel::PanelStaged) {
        if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
            return launch_panel_staged<Fmt::Q8_0, Mode::Plain>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        if (fmt == Fmt::Q4 && mode == Mode::Plain)
            return launch_panel_staged<Fmt::Q4, Mode::Plain>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
            return launch_panel_staged<Fmt::Q4, Mode::SwiGLU>(wa, sa, wb, sb, xq, xd, y, m, n, k, stream);
        return hipErrorInvalidValue;
    }
    if (p.kernel != plan::Q8Kernel::Dot4)
        return launch_qmm_q8act_mfma(fmt, mode, wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
    const int mt = static_cast<int>(p.mt);
    if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
        return dispatch<Fmt::Q8_0, Mode::Plain>(wa, sa, wb, sb, xq, xd, y, m, n, k, mt, stream);
    if (fmt == Fmt::Q4 && mode == Mode::Plain)
        return dispatch<Fmt::Q4, Mode::Plain>(wa, sa, wb, sb, xq, xd, y, m, n, k, mt, stream);
    if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
        return dispatch<Fmt::Q4, Mode::SwiGLU>(wa, sa, wb, sb, xq, xd, y, m, n, k, mt, stream);
    return hipErrorInvalidValue;
}

// Quantize x and multiply in one call: where the staged M = 1 kernel takes
// the shape and its threads quantize the panel in a few rounds, it does so
// itself (one launch); elsewhere the producer and the product run as two
// launches.  Either way xq, xd and y
// are those of quantize_act_q8_0 followed by launch_qmm_q8act.
hipError_t launch_qmm_q8act_from_f32(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa,
                                     const void* wb, const uint16_t* sb, const float* x, int8_t* xq,
                                     float* xd, float* y, int64_t M, int64_t N, int64_t K,
                                     hipStream_t stream) {
    if (plan::q8act_m1_qx_per_row(fmt, M, N, K, device_cus())) {
        const int n = static_cast<int>(N), k = static_cast<int>(K);
        if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
            return launch_m1_qx<Fmt::Q8_0, Mode::Plain>(wa, sa, wb, sb, x, xq, xd, y, n, k, stream);
        if (fmt == Fmt::Q4 && mode == Mode::Plain)
            return launch_m1_qx<Fmt::Q4, Mode::Plain>(wa, sa, wb, sb, x, xq, xd, y, n, k, stream);
        if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
            return launch_m1_qx<Fmt::Q4, Mode::SwiGLU>(wa, sa, wb, sb, x, xq, xd, y, n, k, stream);
        return hipErrorInvalidValue;
    }
    if (plan::q8act_m1_quantize_inside(fmt, M, N, K, device_cus()))
        return launch_m1_staged_any<true>(fmt, mode, wa, sa, wb, sb, ActIn{nullptr, nullptr, x, xq, xd}, y,
                                          static_cast<int>(N), static_cast<int>(K), stream);
    const hipError_t e = launch_quantize_q8(x, xq, xd, M, K, stream);
    if (e != hipSuccess) return e;
    return launch_qmm_q8act(fmt, mode, wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
}

}  // namespace qbd
