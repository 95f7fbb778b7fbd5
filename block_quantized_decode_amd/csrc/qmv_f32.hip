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
#include <atomic>

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
    __device__ static float scale(uint16_t bits) { return f16_bits_to_f32(bits); }
};

// Q4: chunk c = block c (16 bytes); byte j: code j (low), code j + 16 (high).
template <> struct Chunk<Fmt::Q4> {
    static constexpr int kCodes = 32;
    static constexpr int kMaxJ = 4;
    __device__ static int block_of(int c) { return c; }
    // 16 x the chunk dot (codes as 16 (q - 8)); the block scale is d / 16
    __device__ static float dot(const uint4 w, const float (&xs)[kCodes]) {
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = q4x16_lo(d[i]), hi = q4x16_hi(d[i]);
            t0 = __builtin_fmaf(sbyte_f32<0>(lo), xs[4 * i + 0], t0);
            t1 = __builtin_fmaf(sbyte_f32<0>(hi), xs[16 + 4 * i + 0], t1);
            t0 = __builtin_fmaf(sbyte_f32<1>(lo), xs[4 * i + 1], t0);
            t1 = __builtin_fmaf(sbyte_f32<1>(hi), xs[16 + 4 * i + 1], t1);
            t0 = __builtin_fmaf(sbyte_f32<2>(lo), xs[4 * i + 2], t0);
            t1 = __builtin_fmaf(sbyte_f32<2>(hi), xs[16 + 4 * i + 2], t1);
            t0 = __builtin_fmaf(sbyte_f32<3>(lo), xs[4 * i + 3], t0);
            t1 = __builtin_fmaf(sbyte_f32<3>(hi), xs[16 + 4 * i + 3], t1);
        }
        return t0 + t1;
    }
    __device__ static float scale(uint16_t bits) { return q4_scale(bits); }
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
            const float d = C::scale(rsa[C::block_of(c)]);
            uint4 w2 = make_uint4(0, 0, 0, 0);
            float d2 = 0.f;
            if constexpr (MODE == Mode::SwiGLU) {
                w2 = load_w(rb + static_cast<size_t>(c) * 16);
                d2 = C::scale(rsb[C::block_of(c)]);
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

// M = 1: each lane keeps its K-slice of x in VGPRs; a wave owns R rows and
// keeps R * J 16-byte loads in flight.  No load sits under a per-lane
// branch (that would serialize them): chunk and row indices are clamped to
// valid addresses, and a chunk past the end of K meets a zero x slice, so
// it adds exactly zero.
template <Fmt F, Mode MODE, int J, int R>
__global__ __launch_bounds__(256) void qmv_f32_m1(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int N, int K) {
    using C = Chunk<F>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    const size_t rbytes = row_bytes<F>(K);

    int cj[J];
#pragma unroll
    for (int j = 0; j < J; ++j) cj[j] = min(j * kWave + lane, nchunks - 1);

    const int n0 = (blockIdx.x * 4 + wave) * R;
    if (n0 >= N) return;  // whole wave

    // the row group's weights, issued before anything else
    uint4 wva[R][J], wvb[R][J];
    uint16_t sva[R][J], svb[R][J];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const size_t row = static_cast<size_t>(min(n0 + r, N - 1));
#pragma unroll
        for (int j = 0; j < J; ++j) {
            wva[r][j] = load_w(wa + row * rbytes + static_cast<size_t>(cj[j]) * 16);
            sva[r][j] = sa[row * nblocks + C::block_of(cj[j])];
            if constexpr (MODE == Mode::SwiGLU) {
                wvb[r][j] = load_w(wb + row * rbytes + static_cast<size_t>(cj[j]) * 16);
                svb[r][j] = sb[row * nblocks + C::block_of(cj[j])];
            }
        }
    }

    float xr[J][C::kCodes];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        load_x(x + static_cast<size_t>(cj[j]) * C::kCodes, xr[j]);
        const bool live = j * kWave + lane < nchunks;
#pragma unroll
        for (int i = 0; i < C::kCodes; ++i) xr[j][i] = live ? xr[j][i] : 0.f;
    }

    float acc_a[R], acc_b[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc_a[r] = 0.f;
        acc_b[r] = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            acc_a[r] = __builtin_fmaf(C::scale(sva[r][j]), C::dot(wva[r][j], xr[j]), acc_a[r]);
            if constexpr (MODE == Mode::SwiGLU)
                acc_b[r] = __builtin_fmaf(C::scale(svb[r][j]), C::dot(wvb[r][j], xr[j]), acc_b[r]);
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

// M = 1 with long rows and few of them: one wave per K sweep.  A workgroup
// owns R rows and has J waves; wave j takes chunk j * 64 + lane of each
// row, so every wave waits on one 16-byte weight load per row, and a
// 896-row matrix with 5 sweeps runs 2240 waves (two rows per workgroup)
// instead of 896.  Each wave
// reduces its per-lane terms with the DPP tree, and the J wave sums of a
// row are added in sweep order through LDS: one fixed order per output
// (plain and SwiGLU alike), which differs from the per-row kernels' order.
template <Fmt F, Mode MODE, int R>
__global__ __launch_bounds__(1024) void qmv_f32_m1_sweep(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int N, int K) {
    using C = Chunk<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    __shared__ float part[NMAT][16][R];
    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // sweep of this wave
    const int J = blockDim.x >> 6;
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    const size_t rbytes = row_bytes<F>(K);
    const int c = min(j * kWave + lane, nchunks - 1);
    const bool live = j * kWave + lane < nchunks;
    const int n0 = blockIdx.x * R;
    const uint8_t* const wm[2] = {wa, wb};
    const uint16_t* const sm[2] = {sa, sb};

    uint4 w[NMAT][R];
    uint16_t sc[NMAT][R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const size_t row = static_cast<size_t>(min(n0 + r, N - 1));
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            w[q][r] = load_w(wm[q] + row * rbytes + static_cast<size_t>(c) * 16);
            sc[q][r] = sm[q][row * nblocks + C::block_of(c)];
        }
    }
    float xs[C::kCodes];
    load_x(x + static_cast<size_t>(c) * C::kCodes, xs);
#pragma unroll
    for (int i = 0; i < C::kCodes; ++i) xs[i] = live ? xs[i] : 0.f;

#pragma unroll
    for (int q = 0; q < NMAT; ++q) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(C::scale(sc[q][r]), C::dot(w[q][r], xs), 0.f);
        wave_reduce<R>(acc);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (lane == reduced_lane<R>(r)) part[q][j][r] = acc[r];
    }
    __syncthreads();
    if (threadIdx.x < R && n0 + static_cast<int>(threadIdx.x) < N) {
        const int r = threadIdx.x;
        float v[NMAT];
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
            float t = part[q][0][r];
            for (int k = 1; k < J; ++k) t += part[q][k][r];
            v[q] = t;
        }
        y[n0 + r] = MODE == Mode::SwiGLU ? swiglu_f32(v[0], v[NMAT - 1]) : v[0];
    }
}

// Row of a wave_reduce<R> result held by this lane (every lane holds one).
template <int R>
__device__ __forceinline__ int lane_row(int lane) {
    if constexpr (R == 1) return 0;
    else if constexpr (R == 2) return lane >> 5;
    else return (lane & 16 ? 2 : 0) + (lane >> 5);  // R == 4: {0, 2, 1, 3} by 16-lane row
}

// M = 1 over many rows: a persistent grid (as many waves as fit on the
// chip) walks row groups with two fixed register sets, so the next group's
// weights are in flight while the current group is converted, reduced and
// stored.  Rows past the end are clamped to the last row, so every load and
// store is unconditional: a clamped group recomputes the last row's value
// with the same arithmetic and stores the same bits to it.  The per-row
// arithmetic is that of qmv_f32_m1, so both kernels give the same bits.
template <Fmt F, Mode MODE, int J, int R>
__global__ __launch_bounds__(256) void qmv_f32_m1_pipe(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int N, int K) {
    using C = Chunk<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    const size_t rbytes = row_bytes<F>(K);
    const uint8_t* const wm[2] = {wa, wb};
    const uint16_t* const sm[2] = {sa, sb};

    int cj[J];
#pragma unroll
    for (int j = 0; j < J; ++j) cj[j] = min(j * kWave + lane, nchunks - 1);

    const int stride = gridDim.x * 4 * R;
    int n0 = (blockIdx.x * 4 + wave) * R;
    if (n0 >= N) return;  // whole wave

    struct Set {
        uint4 w[NMAT][R][J];
        uint16_t s[NMAT][R][J];
    };
    Set A, B;
    auto issue = [&](Set& st, int base) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t row = static_cast<size_t>(min(base + r, N - 1));
#pragma unroll
            for (int q = 0; q < NMAT; ++q) {
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    st.w[q][r][j] = load_w(wm[q] + row * rbytes + static_cast<size_t>(cj[j]) * 16);
                    st.s[q][r][j] = sm[q][row * nblocks + C::block_of(cj[j])];
                }
            }
        }
    };
    issue(A, n0);

    float xr[J][C::kCodes];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        load_x(x + static_cast<size_t>(cj[j]) * C::kCodes, xr[j]);
        const bool live = j * kWave + lane < nchunks;
#pragma unroll
        for (int i = 0; i < C::kCodes; ++i) xr[j][i] = live ? xr[j][i] : 0.f;
    }

    auto consume = [&](const Set& st, int base) {
        float acc[NMAT][R];
#pragma unroll
        for (int q = 0; q < NMAT; ++q) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                acc[q][r] = 0.f;
#pragma unroll
                for (int j = 0; j < J; ++j)
                    acc[q][r] = __builtin_fmaf(C::scale(st.s[q][r][j]), C::dot(st.w[q][r][j], xr[j]), acc[q][r]);
            }
            wave_reduce<R>(acc[q]);
        }
        // every lane holds the total of row lane_row<R>(lane); the value
        // is the same in all lanes that write one address
        const int r = lane_row<R>(lane);
        float out = acc[0][0];
        if constexpr (MODE == Mode::SwiGLU) out = swiglu_f32(acc[0][0], acc[NMAT - 1][0]);
        y[min(base + r, N - 1)] = out;
    };

    for (;;) {
        issue(B, n0 + stride);
        consume(A, n0);
        n0 += stride;
        if (n0 >= N) break;
        issue(A, n0 + stride);
        consume(B, n0);
        n0 += stride;
        if (n0 >= N) break;
    }
}

// M = 1 with long rows.  x is staged once per workgroup (one per CU) in
// LDS, part-major, and each lane reads the kCodes x values of its chunk for
// one sweep from there; weight chunks and the per-lane accumulation are
// those of qmv_f32_m1 (chunk c = j * 64 + lane, blocks in sweep order, the
// same DPP tree), so both kernels give the same bits.  A workgroup owns a
// contiguous range of rows; wave w takes rows row_begin + R (w + 16 g).
// Items are (row group, sweep) pairs; two register sets A and B hold the
// weight chunks of alternate items, so the next item's loads are in flight
// while the current one is multiplied.  Loads are unconditional (clamped
// rows and chunks, in bounds) and outputs go to LDS and out at the end: a
// load or a store under the loop's branches would make the compiler wait
// for every load in flight.
template <Fmt F, Mode MODE, int R>
__global__ __launch_bounds__(1024) void qmv_f32_m1_staged(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int N, int K, int J, int rows_per_wg) {
    using C = Chunk<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int P = C::kCodes / 4;  // float4 parts of a chunk's x slice
    extern __shared__ __align__(16) float lds_m1[];
    float4* xq4 = reinterpret_cast<float4*>(lds_m1);                    // [J][P][64]
    float* yout = lds_m1 + static_cast<size_t>(J) * P * kWave * 4;     // [rows_per_wg]
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunks = K / C::kCodes;
    const int nblocks = K / kBlock;
    const size_t rbytes = row_bytes<F>(K);

    // stage x: quad (j, p, l) = x values 4p .. 4p+3 of chunk j * 64 + l
    for (int i = tid; i < K / 4; i += 1024) {
        const int k = 4 * i, c = k / C::kCodes, p = (k % C::kCodes) / 4;
        xq4[((c / kWave) * P + p) * kWave + c % kWave] = *reinterpret_cast<const float4*>(x + k);
    }
    for (int c = nchunks + tid / P; c < J * kWave; c += 1024 / P)  // zero past K
        xq4[((c / kWave) * P + tid % P) * kWave + c % kWave] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    const int row_begin = blockIdx.x * rows_per_wg;
    const int row_end = min(row_begin + rows_per_wg, N);
    const int groups_total = (row_end - row_begin + R - 1) / R;
    const int my_groups = groups_total > wave ? (groups_total - wave + 15) / 16 : 0;
    const int items = my_groups * J;

    struct Slot {
        uint4 w[NMAT][R];
        uint16_t s[NMAT][R];
    };
    int ij = 0, ig = 0;  // sweep and group of the next item to load
    auto issue = [&](Slot& S) {
        const int base = row_begin + R * (wave + 16 * ig);
        const int c = min(ij * kWave + lane, nchunks - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t row = static_cast<size_t>(min(base + r, row_end - 1));
            S.w[0][r] = load_w(wa + row * rbytes + static_cast<size_t>(c) * 16);
            S.s[0][r] = sa[row * nblocks + C::block_of(c)];
            if constexpr (NMAT == 2) {
                S.w[NMAT - 1][r] = load_w(wb + row * rbytes + static_cast<size_t>(c) * 16);
                S.s[NMAT - 1][r] = sb[row * nblocks + C::block_of(c)];
            }
        }
        if (++ij == J) { ij = 0; ++ig; }
    };

    float acc[NMAT][R];
    int j = 0, g = 0;  // sweep and group of the item being multiplied
    auto compute = [&](const Slot& S) {
        if (j == 0) {
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
#pragma unroll
                for (int r = 0; r < R; ++r) acc[q][r] = 0.f;
        }
        float xs[C::kCodes];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const float4 v = xq4[(j * P + p) * kWave + lane];
            xs[4 * p + 0] = v.x; xs[4 * p + 1] = v.y; xs[4 * p + 2] = v.z; xs[4 * p + 3] = v.w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
                acc[q][r] = __builtin_fmaf(C::scale(S.s[q][r]), C::dot(S.w[q][r], xs), acc[q][r]);
        if (j == J - 1) {
            const int base = row_begin + R * (wave + 16 * g);
            wave_reduce<R>(acc[0]);
            if constexpr (NMAT == 2) wave_reduce<R>(acc[NMAT - 1]);
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (lane == reduced_lane<R>(r) && base + r < row_end)
                    yout[base + r - row_begin] =
                        MODE == Mode::SwiGLU ? swiglu_f32(acc[0][r], acc[NMAT - 1][r]) : acc[0][r];
        }
        if (++j == J) { j = 0; ++g; }
    };

    Slot A, B;
    issue(A);
    for (int t = 0; t < items; t += 2) {
        issue(B);  // item t + 1
        compute(A);
        issue(A);  // item t + 2
        if (t + 1 < items) compute(B);
    }

    __syncthreads();
    for (int i = tid; i < row_end - row_begin; i += 1024) y[row_begin + i] = yout[i];
}

// Panels of 2..MT activation rows (MT = 4 or 8).  A lane owns a 16-code
// chunk of K (Q8_0: 16 bytes, Q4: 8 bytes = half a block: codes 8h..8h+7
// and 16+8h..16+8h+7 of its block) for each of the wave's rows; the x panel
// sits in LDS in sweeps of 1024 columns, and each lane reads the 16 x values
// of its chunk for one panel row at a time, reusing its dequantized codes
// across the MT rows.  The partials of all outputs are reduced at the end
// with one transposing DPP / permlane pass.  Per output: chunks in sweep
// order, each a fixed 16-term FMA sequence scaled by its block scale - the
// same in the plain and the SwiGLU kernels, so fused == unfused holds
// bitwise.
template <Fmt F> struct Half;
template <> struct Half<Fmt::Q8_0> {
    __device__ static void load(const uint8_t* row, int c, uint32_t (&w)[4]) {
        const uint4 v = load_w(row + static_cast<size_t>(c) * 16);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
    __device__ static void codes(const uint32_t (&w)[4], float (&f)[16]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[4 * i + 0] = sbyte_f32<0>(w[i]); f[4 * i + 1] = sbyte_f32<1>(w[i]);
            f[4 * i + 2] = sbyte_f32<2>(w[i]); f[4 * i + 3] = sbyte_f32<3>(w[i]);
        }
    }
    __device__ static float scale(uint16_t bits) { return f16_bits_to_f32(bits); }
    __device__ static int block_of(int c) { return c >> 1; }
    // x offsets (in the sweep's LDS row) of the chunk's 16 codes: two runs of 8
    __device__ static int run0(int cl) { return 16 * cl; }
    __device__ static int run1(int cl) { return 16 * cl + 8; }
    // column k -> (chunk, part): part p holds the chunk's codes 4p .. 4p+3
    __device__ static void part_of(int k, int& c, int& p) { c = k >> 4; p = (k >> 2) & 3; }
};
template <> struct Half<Fmt::Q4> {
    __device__ static void load(const uint8_t* row, int c, uint32_t (&w)[4]) {
        const uint2 v = *reinterpret_cast<const uint2*>(row + static_cast<size_t>(c) * 8);
        w[0] = v.x; w[1] = v.y; w[2] = 0; w[3] = 0;
    }
    // 16 (q - 8) per code; the block scale is d / 16
    __device__ static void codes(const uint32_t (&w)[4], float (&f)[16]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t lo = q4x16_lo(w[i]), hi = q4x16_hi(w[i]);
            f[4 * i + 0] = sbyte_f32<0>(lo); f[4 * i + 1] = sbyte_f32<1>(lo);      // codes 8h + 4i + b
            f[4 * i + 2] = sbyte_f32<2>(lo); f[4 * i + 3] = sbyte_f32<3>(lo);
            f[8 + 4 * i + 0] = sbyte_f32<0>(hi); f[8 + 4 * i + 1] = sbyte_f32<1>(hi);  // codes 16 + 8h + 4i + b
            f[8 + 4 * i + 2] = sbyte_f32<2>(hi); f[8 + 4 * i + 3] = sbyte_f32<3>(hi);
        }
    }
    __device__ static float scale(uint16_t bits) { return q4_scale(bits); }
    __device__ static int block_of(int c) { return c >> 1; }
    __device__ static int run0(int cl) { return 32 * (cl >> 1) + 8 * (cl & 1); }
    __device__ static int run1(int cl) { return 32 * (cl >> 1) + 16 + 8 * (cl & 1); }
    // column k -> (chunk, part): a chunk's codes are 8h..8h+7 then 16+8h..16+8h+7
    // of its block; part p holds codes 4p .. 4p+3 of that order
    __device__ static void part_of(int k, int& c, int& p) {
        const int b = k >> 5, r = k & 31;
        const int hi = r >> 4, h = (r >> 3) & 1;
        c = 2 * b + h;
        p = 2 * hi + ((r >> 2) & 1);
    }
};

__device__ __forceinline__ float dot16(const float (&w)[16], const float (&xv)[16]) {
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        t0 = __builtin_fmaf(w[i], xv[i], t0);
        t1 = __builtin_fmaf(w[i + 1], xv[i + 1], t1);
    }
    return t0 + t1;
}

constexpr int kPanelKC = static_cast<int>(plan::kPanelKC);  // columns of K per sweep (64 lanes x 16 codes)

// Panels whose x fits in LDS whole (MT * K * 4 bytes): one 1024-thread
// workgroup per CU stages the panel once, then its 16 waves walk their own
// groups of R output rows over the full K, the weight chunks of the next
// items in flight while the current one is multiplied.  Same per-output
// order as qmv_f32_panel_chunked (chunks in sweep order, dot16, block scale,
// one transposing reduction), so either kernel gives the same bits for a
// given output.  Sixteen waves per CU (128 VGPRs each) beat fewer, wider
// waves here: with eight waves and twice the rows per x read, or four waves
// and four times, the kernel ran 10% and 60% slower.
// YLDS: outputs are gathered in LDS behind the panel and written once at
// the end (set when the LDS has room for them).  A global store inside the
// item loop, under its branches, makes the compiler wait for every load in
// flight at the top of each unrolled round.
template <Fmt F, Mode MODE, int MT, int R, bool YLDS>
__global__ __launch_bounds__(1024) void qmv_f32_panel_resident(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int M, int N, int K, int J, int rows_per_wg) {
    using H = Half<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int MTP = (MT + 3) / 4 * 4;
    constexpr int NVP = NMAT * MTP;
    // [MT][J][4][64] float4 quads of x, then [MT][rows_per_wg] outputs
    extern __shared__ __align__(16) float xs_all[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = blockIdx.y * MT;
    const int nchunks = K / 16;
    const int nblocks = K / kBlock;
    const size_t rbytes = row_bytes<F>(K);
    float* yout = xs_all + static_cast<size_t>(MT) * J * kPanelKC;

    // Stage the panel, part-major: quad (m, j, p, cl) holds x values 4p .. 4p+3
    // of chunk cl of sweep j for row m, so the 64 lanes of one 16-byte LDS
    // read touch 64 consecutive quads (no bank conflicts).  Rows past M and
    // columns past K are zero.
    float4* xq4 = reinterpret_cast<float4*>(xs_all);
    const int quads = MT * (K / 4);
    for (int i = tid; i < quads; i += 1024) {
        const int m = i / (K / 4), k = 4 * (i % (K / 4));
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m0 + m < M) v = *reinterpret_cast<const float4*>(x + static_cast<size_t>(m0 + m) * K + k);
        int c, p;
        H::part_of(k, c, p);
        xq4[((m * J + c / kWave) * 4 + p) * kWave + c % kWave] = v;
    }
    if (nchunks % kWave != 0) {  // zero the tail of the last sweep
        const int tail = kWave - nchunks % kWave;
        for (int i = tid; i < MT * 4 * tail; i += 1024) {
            const int m = i / (4 * tail), r = i % (4 * tail);
            xq4[((m * J + J - 1) * 4 + r / tail) * kWave + kWave - tail + r % tail] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    __syncthreads();

    // Items are (row group, sweep) pairs of this wave, group-major: group g
    // holds rows row_begin + R * (wave + 16 g) .. + R - 1 (clamped).  An item
    // reads its x slices from LDS once for the R rows.  Weight chunks are
    // loaded PD items ahead into a ring of registers (static slots: the loop
    // is unrolled by PD).  Sweep and group of the item being multiplied and
    // of the item being loaded are kept as running counters.
    constexpr int PD = 4;
    const int row_begin = blockIdx.x * rows_per_wg;
    const int row_end = min(row_begin + rows_per_wg, N);
    const int groups_total = (row_end - row_begin + R - 1) / R;
    const int my_groups = groups_total > wave ? (groups_total - wave + 15) / 16 : 0;
    const int items = my_groups * J;
    uint32_t raw[PD][NMAT][R][4];
    uint16_t sraw[PD][NMAT][R];
    int ij = 0, ig = 0;  // sweep and group of the next item to load
    auto issue = [&](uint32_t (&rw)[NMAT][R][4], uint16_t (&sr)[NMAT][R]) {
        const int base = row_begin + R * (wave + 16 * ig);
        const int c = min(ij * kWave + lane, nchunks - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t row = static_cast<size_t>(min(base + r, row_end - 1));
            H::load(wa + row * rbytes, c, rw[0][r]);
            sr[0][r] = sa[row * nblocks + H::block_of(c)];
            if constexpr (NMAT == 2) {
                H::load(wb + row * rbytes, c, rw[1][r]);
                sr[1][r] = sb[row * nblocks + H::block_of(c)];
            }
        }
        if (++ij == J) { ij = 0; ++ig; }
    };
    // loads are issued unconditionally (past the last item they repeat
    // clamped rows and chunks, in bounds and unused): a load under a branch
    // would make the compiler merge the ring slots and wait on every load
#pragma unroll
    for (int u = 0; u < PD; ++u) issue(raw[u], sraw[u]);

    float acc[NMAT][R][MT];
    int j = 0, g = 0;  // sweep and group of the item being multiplied
    for (int t0 = 0; t0 < items; t0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int t = t0 + u;
            if (t < items) {
                if (j == 0) {
#pragma unroll
                    for (int q = 0; q < NMAT; ++q)
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int m = 0; m < MT; ++m) acc[q][r][m] = 0.f;
                }
                const int c = j * kWave + lane;
                const bool live = c < nchunks;
                const int cl = min(c, nchunks - 1) - j * kWave;  // chunk within the sweep
                float w[NMAT][R][16];
                float d[NMAT][R];
#pragma unroll
                for (int q = 0; q < NMAT; ++q)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        H::codes(raw[u][q][r], w[q][r]);
                        const float dv = H::scale(sraw[u][q][r]);
                        d[q][r] = live ? dv : 0.f;  // a chunk past K adds exactly zero
                    }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float4* xr = xq4 + (m * J + j) * 4 * kWave + cl;
                    float xv[16];
                    const float4 a0 = xr[0];
                    const float4 a1 = xr[kWave];
                    const float4 a2 = xr[2 * kWave];
                    const float4 a3 = xr[3 * kWave];
                    xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
                    xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
                    xv[8] = a2.x; xv[9] = a2.y; xv[10] = a2.z; xv[11] = a2.w;
                    xv[12] = a3.x; xv[13] = a3.y; xv[14] = a3.z; xv[15] = a3.w;
#pragma unroll
                    for (int q = 0; q < NMAT; ++q)
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[q][r][m] = __builtin_fmaf(d[q][r], dot16(w[q][r], xv), acc[q][r][m]);
                }
                if (j == J - 1) {
                    const int base = row_begin + R * (wave + 16 * g);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        // each matrix's MT values padded to a multiple of 4, so
                        // the gate and up sums of row m end in the same lane
                        float flat[NVP];
#pragma unroll
                        for (int v = 0; v < NVP; ++v) flat[v] = 0.f;
#pragma unroll
                        for (int q = 0; q < NMAT; ++q)
#pragma unroll
                            for (int m = 0; m < MT; ++m) flat[q * MTP + m] = acc[q][r][m];
                        float red[NVP / 4];
                        wave_reduce_many<NVP>(flat, red);
                        const int n = base + r;
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            if (lane == many_lane(m % 4) && n < row_end) {
                                const float gv = red[m / 4];
                                const float out = MODE == Mode::SwiGLU ? swiglu_f32(gv, red[(m + MTP) / 4]) : gv;
                                if constexpr (YLDS) yout[m * rows_per_wg + (n - row_begin)] = out;
                                else if (m0 + m < M) y[static_cast<size_t>(m0 + m) * N + n] = out;
                            }
                        }
                    }
                }
                if (++j == J) { j = 0; ++g; }
            }
            issue(raw[u], sraw[u]);  // item t + PD
            // keep the unrolled items apart: merged, their loads and x slices
            // would not fit in the register file
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if constexpr (YLDS) {  // coalesced write-out of the gathered outputs
        __syncthreads();
        const int nrows = row_end - row_begin;
        for (int i = tid; i < MT * nrows; i += 1024) {
            const int m = i / nrows, r = i % nrows;
            if (m0 + m < M) y[static_cast<size_t>(m0 + m) * N + row_begin + r] = yout[m * rows_per_wg + r];
        }
    }
}

// Panels whose x does not fit in LDS (long rows: K above 5120 for 8 rows).
// x streams through LDS in chunks of JC sweeps (double buffered), and each
// wave keeps its rows - at most RMAX, rows row_begin + w + 16 i - for the
// whole of K, so its per-lane accumulators stay in registers across chunks.
// Per lane and output, sweeps are taken in order, each a fixed 16-term FMA
// sequence scaled by its block scale, then the same DPP tree: the same bits
// as the resident kernel.  The next chunk's x and weights are loaded into
// fixed register sets (the chunk loop is unrolled by two) while the current
// chunk is multiplied; every load is unconditional (clamped, in bounds), and
// the only global stores come after the loop.
template <Fmt F, Mode MODE, int MT, int JC, int RMAX>
__global__ __launch_bounds__(1024) void qmv_f32_panel_chunked(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const float* __restrict__ x, float* __restrict__ y, int M, int N, int K, int rows_per_wg) {
    using H = Half<F>;
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int MTP = (MT + 3) / 4 * 4;
    constexpr int NVP = NMAT * MTP;
    constexpr int CQ = MT * JC * (kPanelKC / 4);  // float4 quads of x per chunk
    constexpr int QT = CQ / 1024;                 // per thread
    static_assert(CQ % 1024 == 0, "whole quads per thread");
    extern __shared__ __align__(16) float xs_chunk[];  // 2 x [MT][JC][4][64] float4
    float4* xbuf = reinterpret_cast<float4*>(xs_chunk);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = blockIdx.y * MT;
    const int nchunks = K / 16;                 // 16-code chunks of a row
    const int nblocks = K / kBlock;
    const int J = (nchunks + kWave - 1) / kWave;
    const int NC = (J + JC - 1) / JC;           // K chunks
    const size_t rbytes = row_bytes<F>(K);
    const int row_begin = blockIdx.x * rows_per_wg;
    const int row_end = min(row_begin + rows_per_wg, N);
    const int nr = row_end - row_begin > wave ? (row_end - row_begin - wave + 15) / 16 : 0;  // my rows (<= RMAX)

    // ---- x chunk: global -> registers -> LDS (part-major per sweep, zero past K / M)
    float4 xr[QT];
    auto xload = [&](int c) {
        const int cc = min(c, NC - 1);
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            const int i = tid + 1024 * u;
            const int m = i / (JC * kPanelKC / 4), kk = 4 * (i % (JC * kPanelKC / 4));
            const int k = cc * JC * kPanelKC + kk;
            const int mm = min(m0 + m, M - 1), kc = min(k, K - 4);
            xr[u] = *reinterpret_cast<const float4*>(x + static_cast<size_t>(mm) * K + kc);
        }
    };
    auto xstore = [&](int c, int buf) {
        float4* xb = xbuf + buf * CQ;
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            const int i = tid + 1024 * u;
            const int m = i / (JC * kPanelKC / 4), kk = 4 * (i % (JC * kPanelKC / 4));
            const int k = c * JC * kPanelKC + kk;
            const bool live = m0 + m < M && k < K;
            int cl, p;
            H::part_of(kk, cl, p);  // cl: chunk within the JC sweeps of this buffer
            xb[((m * JC + cl / kWave) * 4 + p) * kWave + cl % kWave] = live ? xr[u] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };

    // ---- weights of a K chunk for this wave's rows
    struct WSet {
        uint32_t raw[RMAX][JC][NMAT][4];
        uint16_t sc[RMAX][JC][NMAT];
    };
    auto wload = [&](WSet& W, int c) {
        const int cc = min(c, NC - 1);
#pragma unroll
        for (int i = 0; i < RMAX; ++i) {
            const size_t row = static_cast<size_t>(min(row_begin + wave + 16 * i, row_end - 1));
#pragma unroll
            for (int jj = 0; jj < JC; ++jj) {
                const int ch = min((cc * JC + jj) * kWave + lane, nchunks - 1);
                H::load(wa + row * rbytes, ch, W.raw[i][jj][0]);
                W.sc[i][jj][0] = sa[row * nblocks + H::block_of(ch)];
                if constexpr (NMAT == 2) {
                    H::load(wb + row * rbytes, ch, W.raw[i][jj][NMAT - 1]);
                    W.sc[i][jj][NMAT - 1] = sb[row * nblocks + H::block_of(ch)];
                }
            }
        }
    };

    float acc[RMAX][NMAT][MT];
#pragma unroll
    for (int i = 0; i < RMAX; ++i)
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[i][q][m] = 0.f;

    auto compute = [&](const WSet& W, int c, int buf) {
        const float4* xb = xbuf + buf * CQ;
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
            const int j = c * JC + jj;  // sweep
            if (j < J) {                // wave-uniform
                const int ch = j * kWave + lane;
                const bool live = ch < nchunks;
                const int cl = min(ch, nchunks - 1) - j * kWave;
#pragma unroll
                for (int i = 0; i < RMAX; ++i) {
                    if (i < nr) {  // wave-uniform
                        float w[NMAT][16];
                        float d[NMAT];
#pragma unroll
                        for (int q = 0; q < NMAT; ++q) {
                            H::codes(W.raw[i][jj][q], w[q]);
                            const float dv = H::scale(W.sc[i][jj][q]);
                            d[q] = live ? dv : 0.f;  // a chunk past K adds exactly zero
                        }
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            const float4* xq = xb + (m * JC + jj) * 4 * kWave + cl;
                            float xv[16];
                            const float4 a0 = xq[0], a1 = xq[kWave], a2 = xq[2 * kWave], a3 = xq[3 * kWave];
                            xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
                            xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
                            xv[8] = a2.x; xv[9] = a2.y; xv[10] = a2.z; xv[11] = a2.w;
                            xv[12] = a3.x; xv[13] = a3.y; xv[14] = a3.z; xv[15] = a3.w;
#pragma unroll
                            for (int q = 0; q < NMAT; ++q)
                                acc[i][q][m] = __builtin_fmaf(d[q], dot16(w[q], xv), acc[i][q][m]);
                        }
                    }
                }
            }
        }
    };

    WSet A, B;
    xload(0);
    wload(A, 0);
    xstore(0, 0);
    __syncthreads();
    for (int c = 0; c < NC; c += 2) {
        xload(c + 1);
        wload(B, c + 1);
        compute(A, c, 0);
        xstore(c + 1, 1);  // buffer 1 was last read before the previous barrier
        __syncthreads();
        if (c + 1 < NC) {  // uniform across the workgroup
            xload(c + 2);
            wload(A, c + 2);
            compute(B, c + 1, 1);
            xstore(c + 2, 0);
            __syncthreads();
        }
    }

    // ---- reduce and store this wave's rows
#pragma unroll
    for (int i = 0; i < RMAX; ++i) {
        if (i < nr) {
            float flat[NVP];
#pragma unroll
            for (int v = 0; v < NVP; ++v) flat[v] = 0.f;
#pragma unroll
            for (int q = 0; q < NMAT; ++q)
#pragma unroll
                for (int m = 0; m < MT; ++m) flat[q * MTP + m] = acc[i][q][m];
            float red[NVP / 4];
            wave_reduce_many<NVP>(flat, red);
            const int n = row_begin + wave + 16 * i;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (lane == many_lane(m % 4) && m0 + m < M) {
                    const float gv = red[m / 4];
                    y[static_cast<size_t>(m0 + m) * N + n] =
                        MODE == Mode::SwiGLU ? swiglu_f32(gv, red[(m + MTP) / 4]) : gv;
                }
            }
        }
    }
}

constexpr size_t kLdsBytes = static_cast<size_t>(plan::kLdsBytes);

// Sweeps of the staged panel: 1024 columns each (64 lanes x 16 codes).
inline int panel_sweeps(int K) { return static_cast<int>(plan::panel_sweeps(K)); }

// Rows per workgroup of the resident kernel: one workgroup per CU.
inline int resident_rows(int N) { return static_cast<int>(plan::resident_rows(N, device_cus())); }

// LDS of the resident kernel: the staged panel, plus the outputs of its
// rows when they are gathered in LDS.
inline size_t resident_lds_bytes(int MT, int K, int rows_per_wg, bool ylds) {
    return static_cast<size_t>(plan::resident_lds_bytes(MT, K, rows_per_wg, ylds));
}

template <Fmt F>
inline int m1_sweeps(int K) { return static_cast<int>(plan::m1_sweeps(F, K)); }

template <Fmt F>
inline size_t m1_staged_lds_bytes(int K, int rows_per_wg) {
    return static_cast<size_t>(plan::m1_staged_lds_bytes(F, K, rows_per_wg));
}

template <Fmt F, Mode MODE>
hipError_t launch_m1_staged(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                            const float* x, float* y, int N, int K, hipStream_t stream) {
    const int J = m1_sweeps<F>(K);
    const int rows_per_wg = resident_rows(N);
    const int gx = (N + rows_per_wg - 1) / rows_per_wg;
    const size_t lds = m1_staged_lds_bytes<F>(K, rows_per_wg);
    if (lds > kLdsBytes) return hipErrorInvalidValue;
    // one weight row per item: the finest balance of rows over the waves
    constexpr int R = 1;
    hipLaunchKernelGGL((qmv_f32_m1_staged<F, MODE, R>), dim3(gx), dim3(1024), lds, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                       x, y, N, K, J, rows_per_wg);
    return hipGetLastError();
}

template <Fmt F, Mode MODE, int MT>
hipError_t launch_resident(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                           const float* x, float* y, int M, int N, int K, hipStream_t stream) {
    const int groups = (M + MT - 1) / MT;
    if (groups > 65535) return hipErrorInvalidValue;
    const int J = panel_sweeps(K);
    // one workgroup per CU and row group, rows split evenly
    const int rows_per_wg = resident_rows(N);
    const int gx = (N + rows_per_wg - 1) / rows_per_wg;
    const bool ylds = resident_lds_bytes(MT, K, rows_per_wg, true) <= kLdsBytes;
    const size_t lds = resident_lds_bytes(MT, K, rows_per_wg, ylds);
    if (lds > kLdsBytes) return hipErrorInvalidValue;
    // two weight rows per item (one per matrix in the SwiGLU mode), so each
    // LDS read of an x slice serves two rows; more would not fit in the 128
    // VGPRs of a 1024-thread workgroup
    constexpr int R = MODE == Mode::SwiGLU ? 1 : 2;
    if (ylds)
        hipLaunchKernelGGL((qmv_f32_panel_resident<F, MODE, MT, R, true>), dim3(gx, groups), dim3(1024), lds,
                           stream, static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                           x, y, M, N, K, J, rows_per_wg);
    else
        hipLaunchKernelGGL((qmv_f32_panel_resident<F, MODE, MT, R, false>), dim3(gx, groups), dim3(1024), lds,
                           stream, static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                           x, y, M, N, K, J, rows_per_wg);
    return hipGetLastError();
}

template <Fmt F, Mode MODE, int MT>
hipError_t launch_chunked(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                          const float* x, float* y, int M, int N, int K, hipStream_t stream) {
    const int groups = (M + MT - 1) / MT;
    if (groups > 65535) return hipErrorInvalidValue;
    // chunks of JC sweeps of x per buffer (one where the weight registers
    // of two chunks would not fit next to the accumulators: 16-byte Q8_0
    // chunks, or two matrices); rows: at most RMAX per wave, and at least
    // one workgroup per CU when there are rows for it
    constexpr int JC = F == Fmt::Q8_0 || MODE == Mode::SwiGLU ? 1 : 2;
    constexpr int RMAX = MODE == Mode::SwiGLU ? 1 : 2;
    const int rows_per_wg = max(1, min(16 * RMAX, (N + device_cus() - 1) / device_cus()));
    const int gx = (N + rows_per_wg - 1) / rows_per_wg;
    const size_t lds = 2 * static_cast<size_t>(MT) * JC * kPanelKC * sizeof(float);
    hipLaunchKernelGGL((qmv_f32_panel_chunked<F, MODE, MT, JC, RMAX>), dim3(gx, groups), dim3(1024), lds, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                       x, y, M, N, K, rows_per_wg);
    return hipGetLastError();
}


template <Fmt F, Mode MODE, int J, int R>
hipError_t launch_m1(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                     const float* x, float* y, int N, int K, hipStream_t stream) {
    const int blocks = ((N + R - 1) / R + 3) / 4;
    hipLaunchKernelGGL((qmv_f32_m1<F, MODE, J, R>), dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                       x, y, N, K);
    return hipGetLastError();
}

// A persistent grid: as many 256-thread workgroups as are resident at once.
template <Fmt F, Mode MODE, int J, int R>
hipError_t launch_m1_pipe(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                          const float* x, float* y, int N, int K, hipStream_t stream) {
    static const int per_cu = [] {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, qmv_f32_m1_pipe<F, MODE, J, R>, 256, 0) !=
                hipSuccess || v < 1)
            v = 4;
        return v;
    }();
    const int blocks = ((N + R - 1) / R + 3) / 4;
    const int grid = min(blocks, per_cu * device_cus());
    hipLaunchKernelGGL((qmv_f32_m1_pipe<F, MODE, J, R>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb,
                       x, y, N, K);
    return hipGetLastError();
}


template <Fmt F, Mode MODE, int J>
hipError_t launch_m1_rows(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                          const float* x, float* y, int N, int K, hipStream_t stream) {
    // Many rows: the persistent grid, with as many rows per wave as its two
    // register sets hold at full occupancy (four rows of one 16-byte chunk
    // keep eight loads in flight per lane).
    constexpr int NMAT = MODE == Mode::SwiGLU ? 2 : 1;
    constexpr int RP = J * NMAT == 1 ? 4 : (J * NMAT == 2 ? 2 : 1);
    if (N > plan::kM1PipeMinRows) return launch_m1_pipe<F, MODE, J, RP>(wa, sa, wb, sb, x, y, N, K, stream);
    // Otherwise one row group per wave: two rows once there are enough
    // rows to fill the chip (two 16-byte loads in flight per lane per K
    // sweep); one row otherwise and for long rows, whose J loads per row
    // already keep the lane busy.
    if constexpr (J <= 4) {
        if (N >= 2048) return launch_m1<F, MODE, J, 2>(wa, sa, wb, sb, x, y, N, K, stream);
    }
    return launch_m1<F, MODE, J, 1>(wa, sa, wb, sb, x, y, N, K, stream);
}

// One workgroup of J waves per R rows (plan::m1_sweep_rows).
template <Fmt F, Mode MODE>
hipError_t launch_m1_sweep(int J, const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                           const float* x, float* y, int N, int K, hipStream_t stream) {
    if (J < 2 || J > 16) return hipErrorInvalidValue;
    if (plan::m1_sweep_rows(N) == 2) {
        hipLaunchKernelGGL((qmv_f32_m1_sweep<F, MODE, 2>), dim3((N + 1) / 2), dim3(64 * J), 0, stream,
                           static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb, x, y, N, K);
    } else {
        hipLaunchKernelGGL((qmv_f32_m1_sweep<F, MODE, 1>), dim3(N), dim3(64 * J), 0, stream,
                           static_cast<const uint8_t*>(wa), sa, static_cast<const uint8_t*>(wb), sb, x, y, N, K);
    }
    return hipGetLastError();
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

// The kernel of plan::f32_plan, which depends on the shape, the format and
// the CU count only: the plain and SwiGLU modes of a shape run the same
// kernel family with the same per-output summation order.
template <Fmt F, Mode MODE>
hipError_t dispatch(const void* wa, const uint16_t* sa, const void* wb, const uint16_t* sb,
                    const float* x, float* y, int M, int N, int K, hipStream_t stream) {
    const plan::F32Plan p = plan::f32_plan(F, M, N, K, device_cus());
    switch (p.kernel) {
        case plan::F32Kernel::M1Vgpr:
            return launch_m1_j<F, MODE>(static_cast<int>(p.sweeps), wa, sa, wb, sb, x, y, N, K, stream);
        case plan::F32Kernel::M1Sweep:
            return launch_m1_sweep<F, MODE>(static_cast<int>(p.sweeps), wa, sa, wb, sb, x, y, N, K, stream);
        case plan::F32Kernel::M1Staged:
            return launch_m1_staged<F, MODE>(wa, sa, wb, sb, x, y, N, K, stream);
        case plan::F32Kernel::Mfma:
            return launch_qmv_f32_mfma(F, MODE, wa, sa, wb, sb, x, y, M, N, K, stream);
        case plan::F32Kernel::Resident:
            if (p.mt == 4) return launch_resident<F, MODE, 4>(wa, sa, wb, sb, x, y, M, N, K, stream);
            return launch_resident<F, MODE, 8>(wa, sa, wb, sb, x, y, M, N, K, stream);
        case plan::F32Kernel::Chunked:
            if (p.mt == 4) return launch_chunked<F, MODE, 4>(wa, sa, wb, sb, x, y, M, N, K, stream);
            return launch_chunked<F, MODE, 8>(wa, sa, wb, sb, x, y, M, N, K, stream);
        case plan::F32Kernel::Generic:
            if (M == 1) return launch_generic<F, MODE, 1>(wa, sa, wb, sb, x, y, M, N, K, stream);
            return launch_generic<F, MODE, 4>(wa, sa, wb, sb, x, y, M, N, K, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int device_cus() {
    static std::atomic<int> cache[128];
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 128) return 256;
    const int known = cache[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

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
    if (fmt == Fmt::Q8_0 && mode == Mode::SwiGLU)
        return dispatch<Fmt::Q8_0, Mode::SwiGLU>(wa, sa, wb, sb, x, y, m, n, k, stream);
    return hipErrorInvalidValue;
}

}  // namespace qbd
