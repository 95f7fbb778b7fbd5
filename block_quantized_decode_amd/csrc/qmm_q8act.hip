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
};

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
    const plan::Q8Plan p = plan::q8act_plan(fmt, M, N, K);
    if (p.kernel == plan::Q8Kernel::Tile16)
        return launch_qmm_q8_tile16(static_cast<const int8_t*>(wa), sa, xq, xd, y, M, N, K, stream);
    if (p.kernel != plan::Q8Kernel::Dot4)
        return launch_qmm_q8act_mfma(fmt, mode, wa, sa, wb, sb, xq, xd, y, M, N, K, stream);
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    const int mt = static_cast<int>(p.mt);
    if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
        return dispatch<Fmt::Q8_0, Mode::Plain>(wa, sa, wb, sb, xq, xd, y, m, n, k, mt, stream);
    if (fmt == Fmt::Q4 && mode == Mode::Plain)
        return dispatch<Fmt::Q4, Mode::Plain>(wa, sa, wb, sb, xq, xd, y, m, n, k, mt, stream);
    if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
        return dispatch<Fmt::Q4, Mode::SwiGLU>(wa, sa, wb, sb, xq, xd, y, m, n, k, mt, stream);
    return hipErrorInvalidValue;
}

}  // namespace qbd
