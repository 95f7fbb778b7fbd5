// Block-quantized weights x fp32 activations on gfx950 (wave64, VALU + DPP).
//
// Q8_0 decode GEMV: the weight blocks stay native (32 int8 codes + one fp16
// scale) and are dequantized in registers, one output row per weight row
// (Lumen v0.2.0 release page, "Phase 7.D - Q8-native fused matmul").  The
// same kernels serve 4-bit blocks (d * (q - 8)) and the gate/up SwiGLU
// consumer that produces silu(x.Wg^T) * (x.Wu^T) from one activation panel
// without a gate temporary (LSE v0.4.16 release page, "Combined M8 Q4
// gate/up execution").
//
// Work split: a wave owns R output rows at a time; each lane owns one
// 16-byte weight chunk per 64-lane sweep of K (Q8_0: 16 codes of a block,
// Q4: a whole block of 32 codes), so every wave load is one contiguous,
// 16-byte-per-lane read of a row.  Per lane, chunks are visited in the
// order c = lane, lane + 64, ...; each chunk's dot is a fixed FMA sequence,
// scaled by its block scale into the lane accumulator; lanes are then
// reduced with a fixed DPP / permlane tree.  All kernels here follow that
// one order, so the plain and the SwiGLU kernels give the same projection
// bits and fused == unfused holds bitwise.
#include "device_common.hpp"
#include "launch.hpp"

namespace qbd {
namespace {

template <Fmt F> struct Chunk;

// Q8_0: chunk c = codes [16c, 16c + 16) of a row, block c / 2.
template <> struct Chunk<Fmt::Q8_0> {
    static constexpr int kCodes = 16;
    static constexpr int kMaxJ = 8;
    __device__ static int block_of(int c) { return c >> 1; }
    __device__ static float dot(const uint4 w, const float (&xs)[kCodes]) {
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t0 = __builtin_fmaf(sbyte_f32<0>(d[i]), xs[4 * i + 0], t0);
            t1 = __builtin_fmaf(sbyte_f32<1>(d[i]), xs[4 * i + 1], t1);
            t0 = __builtin_fmaf(sbyte_f32<2>(d[i]), xs[4 * i + 2], t0);
            t1 = __builtin_fmaf(sbyte_f32<3>(d[i]), xs[4 * i + 3], t1);
        }
        return t0 + t1;
    }
};

// Q4: chunk c = block c (16 bytes); byte j: code j (low), code j + 16 (high).
template <> struct Chunk<Fmt::Q4> {
    static constexpr int kCodes = 32;
    static constexpr int kMaxJ = 4;
    __device__ static int block_of(int c) { return c; }
    __device__ static float dot(const uint4 w, const float (&xs)[kCodes]) {
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                t0 = __builtin_fmaf(q4_lo_f32(d[i], b), xs[4 * i + b], t0);
                t1 = __builtin_fmaf(q4_hi_f32(d[i], b), xs[16 + 4 * i + b], t1);
            }
        }
        return t0 + t1;
    }
};

template <Fmt F>
__device__ __forceinline__ size_t row_bytes(int K) {
    return F == Fmt::Q8_0 ? static_cast<size_t>(K) : static_cast<size_t>(K) / 2;
}

template <int N>
__device__ __forceinline__ void load_x(const float* __restrict__ p, float (&xs)[N]) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(p + 4 * i);
        xs[4 * i + 0] = v.x; xs[4 * i + 1] = v.y; xs[4 * i + 2] = v.z; xs[4 * i + 3] = v.w;
    }
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Weight chunks are read once per call: stream them with a non-temporal load.
__device__ __forceinline__ uint4 load_w(const uint8_t* __restrict__ p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Any M: one output row per wave, MT activation rows per pass, x read from
// global memory (it is small and stays in the caches).
template <Fmt F, Mode MODE, int MT>
__global__ __launch_bounds__(256) void qmv_f32_generic(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int M, int N, int K) {
    using C = Chunk<F>;
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;  // whole wave
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    const uint8_t* ra = wa + static_cast<size_t>(n) * row_bytes<F>(K);
    const uint16_t* rsa = sa + static_cast<size_t>(n) * nblocks;
    const uint8_t* rb = MODE == Mode::SwiGLU ? wb + static_cast<size_t>(n) * row_bytes<F>(K) : nullptr;
    const uint16_t* rsb = MODE == Mode::SwiGLU ? sb + static_cast<size_t>(n) * nblocks : nullptr;

    for (int m0 = blockIdx.y * MT; m0 < M; m0 += gridDim.y * MT) {
        float acc_a[MT], acc_b[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) { acc_a[i] = 0.f; acc_b[i] = 0.f; }
        for (int c = lane; c < nchunks; c += kWave) {
            const uint4 w = load_w(ra + static_cast<size_t>(c) * 16);
            const float d = f16_bits_to_f32(rsa[C::block_of(c)]);
            uint4 w2 = make_uint4(0, 0, 0, 0);
            float d2 = 0.f;
            if constexpr (MODE == Mode::SwiGLU) {
                w2 = load_w(rb + static_cast<size_t>(c) * 16);
                d2 = f16_bits_to_f32(rsb[C::block_of(c)]);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if (m0 + i < M) {
                    float xs[C::kCodes];
                    load_x(x + static_cast<size_t>(m0 + i) * K + static_cast<size_t>(c) * C::kCodes, xs);
                    acc_a[i] = __builtin_fmaf(d, C::dot(w, xs), acc_a[i]);
                    if constexpr (MODE == Mode::SwiGLU)
                        acc_b[i] = __builtin_fmaf(d2, C::dot(w2, xs), acc_b[i]);
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

// M = 1: each lane keeps its K-slice of x in VGPRs for the whole row loop;
// a wave owns R rows per pass and keeps R * J 16-byte loads in flight.
template <Fmt F, Mode MODE, int J, int R>
__global__ __launch_bounds__(256) void qmv_f32_m1(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int N, int K) {
    using C = Chunk<F>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    const size_t rbytes = row_bytes<F>(K);

    float xr[J][C::kCodes];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = j * kWave + lane;
        if (c < nchunks) {
            load_x(x + static_cast<size_t>(c) * C::kCodes, xr[j]);
        } else {
#pragma unroll
            for (int i = 0; i < C::kCodes; ++i) xr[j][i] = 0.f;
        }
    }

    const int nwaves = gridDim.x * 4;
    for (int n0 = (blockIdx.x * 4 + wave) * R; n0 < N; n0 += nwaves * R) {
        uint4 wva[R][J], wvb[R][J];
        uint16_t sva[R][J], svb[R][J];
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int c = j * kWave + lane;
                wva[r][j] = make_uint4(0, 0, 0, 0);
                sva[r][j] = 0;
                wvb[r][j] = make_uint4(0, 0, 0, 0);
                svb[r][j] = 0;
                if (c < nchunks && n0 + r < N) {
                    const size_t row = static_cast<size_t>(n0 + r);
                    wva[r][j] = load_w(wa + row * rbytes + static_cast<size_t>(c) * 16);
                    sva[r][j] = sa[row * nblocks + C::block_of(c)];
                    if constexpr (MODE == Mode::SwiGLU) {
                        wvb[r][j] = load_w(wb + row * rbytes + static_cast<size_t>(c) * 16);
                        svb[r][j] = sb[row * nblocks + C::block_of(c)];
                    }
                }
            }
        }
        float acc_a[R], acc_b[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            acc_a[r] = 0.f;
            acc_b[r] = 0.f;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                if (j * kWave + lane < nchunks) {
                    acc_a[r] = __builtin_fmaf(f16_bits_to_f32(sva[r][j]), C::dot(wva[r][j], xr[j]), acc_a[r]);
                    if constexpr (MODE == Mode::SwiGLU)
                        acc_b[r] = __builtin_fmaf(f16_bits_to_f32(svb[r][j]), C::dot(wvb[r][j], xr[j]), acc_b[r]);
                }
            }
        }
        wave_reduce<R>(acc_a);
        if constexpr (MODE == Mode::SwiGLU) wave_reduce<R>(acc_b);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (lane == reduced_lane<R>(r) && n0 + r < N) {
                y[n0 + r] = MODE == Mode::SwiGLU ? swiglu_f32(acc_a[r], acc_b[r]) : acc_a[r];
            }
        }
    }
}

template <Fmt F, Mode MODE, int J, int R>
hipError_t launch_m1(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                     const float* x, float* y, int N, int K, hipStream_t stream) {
    const int waves = (N + R - 1) / R;
    const int blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((qmv_f32_m1<F, MODE, J, R>), dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                       x, y, N, K);
    return hipGetLastError();
}

template <Fmt F, Mode MODE, int J>
hipError_t launch_m1_rows(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                          const float* x, float* y, int N, int K, hipStream_t stream) {
    // Rows per wave: enough waves to spread small matrices over the chip,
    // more loads in flight per wave for large ones, and at most R * J
    // chunks per lane so the x slice and the loads stay in VGPRs.
    if constexpr (J <= 2) {
        if (N >= 32768) return launch_m1<F, MODE, J, 4>(wa, sa, wb, sb, x, y, N, K, stream);
    }
    if constexpr (J <= 4) {
        if (N >= 4096) return launch_m1<F, MODE, J, 2>(wa, sa, wb, sb, x, y, N, K, stream);
    }
    return launch_m1<F, MODE, J, 1>(wa, sa, wb, sb, x, y, N, K, stream);
}

template <Fmt F, Mode MODE>
hipError_t launch_m1_j(int J, const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                       const float* x, float* y, int N, int K, hipStream_t stream) {
    switch (J) {
        case 1: return launch_m1_rows<F, MODE, 1>(wa, sa, wb, sb, x, y, N, K, stream);
        case 2: return launch_m1_rows<F, MODE, 2>(wa, sa, wb, sb, x, y, N, K, stream);
        case 3: return launch_m1_rows<F, MODE, 3>(wa, sa, wb, sb, x, y, N, K, stream);
        case 4: return launch_m1_rows<F, MODE, 4>(wa, sa, wb, sb, x, y, N, K, stream);
        default: break;
    }
    if constexpr (Chunk<F>::kMaxJ > 4) {
        switch (J) {
            case 5: return launch_m1_rows<F, MODE, 5>(wa, sa, wb, sb, x, y, N, K, stream);
            case 6: return launch_m1_rows<F, MODE, 6>(wa, sa, wb, sb, x, y, N, K, stream);
            case 7: return launch_m1_rows<F, MODE, 7>(wa, sa, wb, sb, x, y, N, K, stream);
            case 8: return launch_m1_rows<F, MODE, 8>(wa, sa, wb, sb, x, y, N, K, stream);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

template <Fmt F, Mode MODE, int MT>
hipError_t launch_generic(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                          const float* x, float* y, int M, int N, int K, hipStream_t stream) {
    const int gx = (N + 3) / 4;
    const int chunks = (M + MT - 1) / MT;
    const int gy = chunks < 65535 ? chunks : 65535;
    hipLaunchKernelGGL((qmv_f32_generic<F, MODE, MT>), dim3(gx, gy), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                       x, y, M, N, K);
    return hipGetLastError();
}

template <Fmt F, Mode MODE>
hipError_t dispatch(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                    const float* x, float* y, int M, int N, int K, hipStream_t stream) {
    using C = Chunk<F>;
    const int nchunks = K / C::kCodes;
    const int J = (nchunks + kWave - 1) / kWave;
    if (M == 1 && J <= C::kMaxJ) return launch_m1_j<F, MODE>(J, wa, sa, wb, sb, x, y, N, K, stream);
    if (M == 1) return launch_generic<F, MODE, 1>(wa, sa, wb, sb, x, y, M, N, K, stream);
    if (M == 2) return launch_generic<F, MODE, 2>(wa, sa, wb, sb, x, y, M, N, K, stream);
    return launch_generic<F, MODE, 4>(wa, sa, wb, sb, x, y, M, N, K, stream);
}

}  // namespace

hipError_t launch_qmv_f32(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa,
                          const void* wb, const uint16_t* sb, const float* x, float* y,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    if (fmt == Fmt::Q8_0 && mode == Mode::Plain)
        return dispatch<Fmt::Q8_0, Mode::Plain>(wa, sa, wb, sb, x, y, m, n, k, stream);
    if (fmt == Fmt::Q4 && mode == Mode::Plain)
        return dispatch<Fmt::Q4, Mode::Plain>(wa, sa, wb, sb, x, y, m, n, k, stream);
    if (fmt == Fmt::Q4 && mode == Mode::SwiGLU)
        return dispatch<Fmt::Q4, Mode::SwiGLU>(wa, sa, wb, sb, x, y, m, n, k, stream);
    return hipErrorInvalidValue;
}

}  // namespace qbd
