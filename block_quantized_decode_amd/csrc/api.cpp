// C ABI of libqbd: host-side validation, then dispatch to the gfx950
// kernels on the caller's stream.  Every check runs before the first HIP
// call, so each error path can be exercised on a machine without a GPU.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/qbd.h"
#include "launch.hpp"

namespace {

// Sizes leave 2^20 of headroom below 2^31: the kernels walk rows and
// groups in 32-bit indices that step past the last row by less than that.
constexpr int64_t kMaxDim = (int64_t{1} << 31) - (int64_t{1} << 20);
constexpr int64_t kMaxPlane = int64_t{1} << 40;

struct Span {
    const void* p;
    int64_t bytes;
};

bool overlaps(Span a, Span b) {
    if (a.bytes <= 0 || b.bytes <= 0) return false;
    const auto a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Sizes: M, N >= 0, K > 0 and a multiple of 32, all at most 2^31 - 2^20,
// and every plane (rows * row bytes) below 2^40 bytes.
int check_mnk(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K <= 0 || K % 32 != 0) return QBD_ERR_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return QBD_ERR_SHAPE;
    if (N > 0 && K > kMaxPlane / 4 / N) return QBD_ERR_SHAPE;
    if (M > 0 && K > kMaxPlane / 4 / M) return QBD_ERR_SHAPE;
    if (M > 0 && N > kMaxPlane / 4 / M) return QBD_ERR_SHAPE;
    return QBD_OK;
}

std::atomic<int> g_device_state[128];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return QBD_ERR_DEVICE;
    }
    if (dev >= 128) return QBD_ERR_DEVICE;
    const int known = g_device_state[dev].load(std::memory_order_relaxed);
    if (known == 1) return QBD_OK;
    if (known == 2) return QBD_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return QBD_ERR_DEVICE;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_device_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? QBD_OK : QBD_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? QBD_OK : QBD_ERR_LAUNCH; }

int64_t q8_row_bytes(int64_t K) { return K; }
int64_t q4_row_bytes(int64_t K) { return K / 2; }
int64_t scale_bytes(int64_t N, int64_t K) { return N * (K / 32) * 2; }

// Shared validation of "weights x activations -> y" calls.
struct MatCall {
    int64_t M, N, K;
    Span w[2], s[2];  // weight planes (1 or 2 matrices)
    int nmat;
    Span x, xs;       // activations (fp32 or codes) and activation scales (q8act)
    Span y;
};

int validate(const MatCall& c, bool q8act) {
    for (int i = 0; i < c.nmat; ++i) {
        if (!c.w[i].p || !c.s[i].p) return QBD_ERR_NULL;
    }
    if (!c.x.p || !c.y.p || (q8act && !c.xs.p)) return QBD_ERR_NULL;
    for (int i = 0; i < c.nmat; ++i) {
        if (!aligned(c.w[i].p, 16) || !aligned(c.s[i].p, 2)) return QBD_ERR_ALIGN;
    }
    if (!aligned(c.x.p, 16) || !aligned(c.y.p, 4)) return QBD_ERR_ALIGN;
    if (q8act && !aligned(c.xs.p, 4)) return QBD_ERR_ALIGN;
    for (int i = 0; i < c.nmat; ++i) {
        if (overlaps(c.y, c.w[i]) || overlaps(c.y, c.s[i])) return QBD_ERR_ALIAS;
    }
    if (overlaps(c.y, c.x) || (q8act && overlaps(c.y, c.xs))) return QBD_ERR_ALIAS;
    return QBD_OK;
}

int run_f32(qbd::Fmt fmt, qbd::Mode mode, const void* wa, const uint16_t* sa, const void* wb,
            const uint16_t* sb, const float* x, float* y, int64_t M, int64_t N, int64_t K,
            qbd_stream_t stream) {
    int st = check_mnk(M, N, K);
    if (st != QBD_OK) return st;
    if (M == 0 || N == 0) return QBD_OK;
    const int64_t rb = fmt == qbd::Fmt::Q8_0 ? q8_row_bytes(K) : q4_row_bytes(K);
    MatCall c{};
    c.M = M; c.N = N; c.K = K;
    c.nmat = mode == qbd::Mode::SwiGLU ? 2 : 1;
    c.w[0] = {wa, N * rb}; c.s[0] = {sa, scale_bytes(N, K)};
    c.w[1] = {wb, N * rb}; c.s[1] = {sb, scale_bytes(N, K)};
    c.x = {x, M * K * 4};
    c.xs = {nullptr, 0};
    c.y = {y, M * N * 4};
    st = validate(c, false);
    if (st != QBD_OK) return st;
    st = check_device();
    if (st != QBD_OK) return st;
    return launched(qbd::launch_qmv_f32(fmt, mode, wa, sa, wb, sb, x, y, M, N, K,
                                        reinterpret_cast<hipStream_t>(stream)));
}

int run_q8act(qbd::Fmt fmt, qbd::Mode mode, const void* wa, const uint16_t* sa, const void* wb,
              const uint16_t* sb, const int8_t* xq, const float* xd, float* y, int64_t M,
              int64_t N, int64_t K, qbd_stream_t stream) {
    int st = check_mnk(M, N, K);
    if (st != QBD_OK) return st;
    if (M == 0 || N == 0) return QBD_OK;
    const int64_t rb = fmt == qbd::Fmt::Q8_0 ? q8_row_bytes(K) : q4_row_bytes(K);
    MatCall c{};
    c.M = M; c.N = N; c.K = K;
    c.nmat = mode == qbd::Mode::SwiGLU ? 2 : 1;
    c.w[0] = {wa, N * rb}; c.s[0] = {sa, scale_bytes(N, K)};
    c.w[1] = {wb, N * rb}; c.s[1] = {sb, scale_bytes(N, K)};
    c.x = {xq, M * K};
    c.xs = {xd, M * (K / 32) * 4};
    c.y = {y, M * N * 4};
    st = validate(c, true);
    if (st != QBD_OK) return st;
    st = check_device();
    if (st != QBD_OK) return st;
    return launched(qbd::launch_qmm_q8act(fmt, mode, wa, sa, wb, sb, xq, xd, y, M, N, K,
                                          reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" int quantize_act_q8_0(const float* x, int8_t* xq, float* xd, int64_t M, int64_t K,
                                 qbd_stream_t stream);

namespace {

// quantize_act_q8_0 and a Q8-activation product in one call: x is read,
// xq / xd (the quantized panel) and y are written.  Every output must be
// disjoint from every input and from the other outputs.
int run_q8act_from_f32(qbd::Fmt fmt, qbd::Mode mode, const void* wa, const uint16_t* sa, const void* wb,
                       const uint16_t* sb, const float* x, int8_t* xq, float* xd, float* y, int64_t M,
                       int64_t N, int64_t K, qbd_stream_t stream) {
    int st = check_mnk(M, N, K);
    if (st != QBD_OK) return st;
    if (M == 0) return QBD_OK;
    // no weight rows: only the quantization runs, and only x, xq, xd are looked at
    if (N == 0) return quantize_act_q8_0(x, xq, xd, M, K, stream);
    const int nmat = mode == qbd::Mode::SwiGLU ? 2 : 1;
    const void* w[2] = {wa, wb};
    const uint16_t* s[2] = {sa, sb};
    for (int i = 0; i < nmat; ++i) {
        if (!w[i] || !s[i]) return QBD_ERR_NULL;
    }
    if (!x || !xq || !xd || !y) return QBD_ERR_NULL;
    for (int i = 0; i < nmat; ++i) {
        if (!aligned(w[i], 16) || !aligned(s[i], 2)) return QBD_ERR_ALIGN;
    }
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(y, 4)) return QBD_ERR_ALIGN;
    const int64_t rb = fmt == qbd::Fmt::Q8_0 ? q8_row_bytes(K) : q4_row_bytes(K);
    const Span outs[3] = {{xq, M * K}, {xd, M * (K / 32) * 4}, {y, M * N * 4}};
    Span ins[5] = {{x, M * K * 4}, {w[0], N * rb}, {s[0], scale_bytes(N, K)}, {nullptr, 0}, {nullptr, 0}};
    if (nmat == 2) {
        ins[3] = {w[1], N * rb};
        ins[4] = {s[1], scale_bytes(N, K)};
    }
    for (const Span& o : outs) {
        for (const Span& i : ins) {
            if (overlaps(o, i)) return QBD_ERR_ALIAS;
        }
    }
    if (overlaps(outs[0], outs[1]) || overlaps(outs[0], outs[2]) || overlaps(outs[1], outs[2])) return QBD_ERR_ALIAS;
    st = check_device();
    if (st != QBD_OK) return st;
    return launched(qbd::launch_qmm_q8act_from_f32(fmt, mode, wa, sa, wb, sb, x, xq, xd, y, M, N, K,
                                                   reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* qbd_status_str(int status) {
    switch (status) {
        case QBD_OK: return "ok";
        case QBD_ERR_NULL: return "null pointer";
        case QBD_ERR_SHAPE: return "invalid shape (negative size, K not a positive multiple of 32, or too large)";
        case QBD_ERR_ALIGN: return "misaligned pointer";
        case QBD_ERR_ALIAS: return "output overlaps an input or another output";
        case QBD_ERR_DEVICE: return "no current HIP device, or it is not a gfx950";
        case QBD_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int qbd_abi_version(void) { return 1; }

int qmv_q8_0_f32(const int8_t* wq, const uint16_t* wd, const float* x, float* y, int64_t M,
                 int64_t N, int64_t K, qbd_stream_t stream) {
    return run_f32(qbd::Fmt::Q8_0, qbd::Mode::Plain, wq, wd, nullptr, nullptr, x, y, M, N, K, stream);
}

int qmv_q4_0_f32(const uint8_t* wq4, const uint16_t* wd, const float* x, float* y, int64_t M,
                 int64_t N, int64_t K, qbd_stream_t stream) {
    return run_f32(qbd::Fmt::Q4, qbd::Mode::Plain, wq4, wd, nullptr, nullptr, x, y, M, N, K, stream);
}

int gate_up_swiglu_q4(const uint8_t* gq, const uint16_t* gd, const uint8_t* uq,
                      const uint16_t* ud, const float* x, float* out, int64_t M, int64_t N,
                      int64_t K, qbd_stream_t stream) {
    return run_f32(qbd::Fmt::Q4, qbd::Mode::SwiGLU, gq, gd, uq, ud, x, out, M, N, K, stream);
}

int gate_up_swiglu_q8_0(const int8_t* gq, const uint16_t* gd, const int8_t* uq,
                        const uint16_t* ud, const float* x, float* out, int64_t M, int64_t N,
                        int64_t K, qbd_stream_t stream) {
    return run_f32(qbd::Fmt::Q8_0, qbd::Mode::SwiGLU, gq, gd, uq, ud, x, out, M, N, K, stream);
}

int qmm_q8_0_q8act(const int8_t* wq, const uint16_t* wd, const int8_t* xq, const float* xd,
                   float* y, int64_t M, int64_t N, int64_t K, qbd_stream_t stream) {
    return run_q8act(qbd::Fmt::Q8_0, qbd::Mode::Plain, wq, wd, nullptr, nullptr, xq, xd, y, M, N,
                     K, stream);
}

int qmm_q4_0_q8act(const uint8_t* wq4, const uint16_t* wd, const int8_t* xq, const float* xd,
                   float* y, int64_t M, int64_t N, int64_t K, qbd_stream_t stream) {
    return run_q8act(qbd::Fmt::Q4, qbd::Mode::Plain, wq4, wd, nullptr, nullptr, xq, xd, y, M, N,
                     K, stream);
}

int gate_up_swiglu_q4_q8act(const uint8_t* gq, const uint16_t* gd, const uint8_t* uq,
                            const uint16_t* ud, const int8_t* xq, const float* xd, float* out,
                            int64_t M, int64_t N, int64_t K, qbd_stream_t stream) {
    return run_q8act(qbd::Fmt::Q4, qbd::Mode::SwiGLU, gq, gd, uq, ud, xq, xd, out, M, N, K,
                     stream);
}

int qmm_q8_0_q8act_from_f32(const int8_t* wq, const uint16_t* wd, const float* x, int8_t* xq, float* xd,
                            float* y, int64_t M, int64_t N, int64_t K, qbd_stream_t stream) {
    return run_q8act_from_f32(qbd::Fmt::Q8_0, qbd::Mode::Plain, wq, wd, nullptr, nullptr, x, xq, xd, y, M, N, K,
                              stream);
}

int qmm_q4_0_q8act_from_f32(const uint8_t* wq4, const uint16_t* wd, const float* x, int8_t* xq, float* xd,
                            float* y, int64_t M, int64_t N, int64_t K, qbd_stream_t stream) {
    return run_q8act_from_f32(qbd::Fmt::Q4, qbd::Mode::Plain, wq4, wd, nullptr, nullptr, x, xq, xd, y, M, N, K,
                              stream);
}

int gate_up_swiglu_q4_q8act_from_f32(const uint8_t* gq, const uint16_t* gd, const uint8_t* uq,
                                     const uint16_t* ud, const float* x, int8_t* xq, float* xd, float* out,
                                     int64_t M, int64_t N, int64_t K, qbd_stream_t stream) {
    return run_q8act_from_f32(qbd::Fmt::Q4, qbd::Mode::SwiGLU, gq, gd, uq, ud, x, xq, xd, out, M, N, K, stream);
}

int quantize_act_q8_0(const float* x, int8_t* xq, float* xd, int64_t M, int64_t K,
                      qbd_stream_t stream) {
    int st = check_mnk(M, 1, K);
    if (st != QBD_OK) return st;
    if (M == 0) return QBD_OK;
    if (!x || !xq || !xd) return QBD_ERR_NULL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 4)) return QBD_ERR_ALIGN;
    const Span sx{x, M * K * 4}, sq{xq, M * K}, sd{xd, M * (K / 32) * 4};
    if (overlaps(sq, sx) || overlaps(sd, sx) || overlaps(sq, sd)) return QBD_ERR_ALIAS;
    st = check_device();
    if (st != QBD_OK) return st;
    return launched(qbd::launch_quantize_q8(x, xq, xd, M, K, reinterpret_cast<hipStream_t>(stream)));
}

int swiglu_f32(const float* g, const float* u, float* out, int64_t n, qbd_stream_t stream) {
    if (n < 0 || n > kMaxPlane / 4) return QBD_ERR_SHAPE;
    if (n == 0) return QBD_OK;
    if (!g || !u || !out) return QBD_ERR_NULL;
    if (!aligned(g, 4) || !aligned(u, 4) || !aligned(out, 4)) return QBD_ERR_ALIGN;
    const Span sg{g, n * 4}, su{u, n * 4}, so{out, n * 4};
    if (overlaps(so, sg) || overlaps(so, su)) return QBD_ERR_ALIAS;
    const int st = check_device();
    if (st != QBD_OK) return st;
    return launched(qbd::launch_swiglu(g, u, out, n, reinterpret_cast<hipStream_t>(stream)));
}

int q8_0_split_blocks(const void* blocks34, int8_t* wq, uint16_t* wd, int64_t N, int64_t K) {
    int st = check_mnk(1, N, K);
    if (st != QBD_OK) return st;
    if (N == 0) return QBD_OK;
    if (!blocks34 || !wq || !wd) return QBD_ERR_NULL;
    const auto* src = static_cast<const uint8_t*>(blocks34);
    const int64_t nb = K / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = src + (n * nb + b) * 34;
            wd[n * nb + b] = static_cast<uint16_t>(blk[0] | (blk[1] << 8));
            std::memcpy(wq + n * K + b * 32, blk + 2, 32);
        }
    }
    return QBD_OK;
}

int q4_0_split_blocks(const void* blocks18, uint8_t* wq4, uint16_t* wd, int64_t N, int64_t K) {
    int st = check_mnk(1, N, K);
    if (st != QBD_OK) return st;
    if (N == 0) return QBD_OK;
    if (!blocks18 || !wq4 || !wd) return QBD_ERR_NULL;
    const auto* src = static_cast<const uint8_t*>(blocks18);
    const int64_t nb = K / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = src + (n * nb + b) * 18;
            wd[n * nb + b] = static_cast<uint16_t>(blk[0] | (blk[1] << 8));
            std::memcpy(wq4 + n * (K / 2) + b * 16, blk + 2, 16);
        }
    }
    return QBD_OK;
}

}  // extern "C"
