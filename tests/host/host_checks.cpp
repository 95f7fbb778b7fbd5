// Host-side checks of libqbd, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py:
//   * the C ABI (api.cpp): argument validation, the device check and the
//     hand-off to the launchers, with stand-ins for the three HIP runtime
//     calls it makes and for the kernel launchers;
//   * the host block split helpers, on buffers of exactly the stated size;
//   * the kernel selection rules of plan.hpp over a sweep of shapes.
// Exits 0 when every check holds; prints the first failure otherwise.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/qbd.h"
#include "../../block_quantized_decode_amd/csrc/launch.hpp"

namespace {

int g_failures = 0;

#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_failures;                                                         \
        }                                                                         \
    } while (0)

// what the last launcher stand-in was handed
struct Launch {
    int which = -1;  // 0 qmv_f32, 1 quantize, 2 qmm_q8act, 3 swiglu
    qbd::Fmt fmt = qbd::Fmt::Q8_0;
    qbd::Mode mode = qbd::Mode::Plain;
    int64_t M = -1, N = -1, K = -1;
    int calls = 0;
} g_last;

const char* g_arch = "gfx950:sramecc+:xnack-";

}  // namespace

// ---- stand-ins for the HIP runtime calls made by api.cpp
extern "C" hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}
extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* p, int) {
    std::memset(p, 0, sizeof(*p));
    std::strncpy(p->gcnArchName, g_arch, sizeof(p->gcnArchName) - 1);
    return hipSuccess;
}
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

// ---- stand-ins for the launchers
namespace qbd {
hipError_t launch_qmv_f32(Fmt fmt, Mode mode, const void*, const uint16_t*, const void*, const uint16_t*,
                          const float*, float*, int64_t M, int64_t N, int64_t K, hipStream_t) {
    g_last = {0, fmt, mode, M, N, K, g_last.calls + 1};
    return hipSuccess;
}
hipError_t launch_quantize_q8(const float*, int8_t*, float*, int64_t M, int64_t K, hipStream_t) {
    g_last = {1, Fmt::Q8_0, Mode::Plain, M, -1, K, g_last.calls + 1};
    return hipSuccess;
}
hipError_t launch_qmm_q8act(Fmt fmt, Mode mode, const void*, const uint16_t*, const void*, const uint16_t*,
                            const int8_t*, const float*, float*, int64_t M, int64_t N, int64_t K, hipStream_t) {
    g_last = {2, fmt, mode, M, N, K, g_last.calls + 1};
    return hipSuccess;
}
hipError_t launch_qmm_q8act_from_f32(Fmt fmt, Mode mode, const void*, const uint16_t*, const void*, const uint16_t*,
                                     const float*, int8_t*, float*, float*, int64_t M, int64_t N, int64_t K,
                                     hipStream_t) {
    g_last = {4, fmt, mode, M, N, K, g_last.calls + 1};
    return hipSuccess;
}
hipError_t launch_swiglu(const float*, const float*, float*, int64_t n, hipStream_t) {
    g_last = {3, Fmt::Q8_0, Mode::Plain, -1, n, -1, g_last.calls + 1};
    return hipSuccess;
}
}  // namespace qbd

namespace {

// placeholder device addresses: far apart, 256-byte aligned, never touched
template <typename T>
T* fake(int i, uintptr_t off = 0) {
    return reinterpret_cast<T*>((uintptr_t{1} << 32) * static_cast<uintptr_t>(i + 1) + off);
}

void check_qmv() {
    auto q8 = [](const int8_t* w, const uint16_t* s, const float* x, float* y, int64_t M, int64_t N, int64_t K) {
        return qmv_q8_0_f32(w, s, x, y, M, N, K, nullptr);
    };
    const int8_t* w = fake<int8_t>(0);
    const uint16_t* s = fake<uint16_t>(1);
    const float* x = fake<float>(2);
    float* y = fake<float>(3);
    EXPECT(q8(w, s, x, y, 1, 64, 48) == QBD_ERR_SHAPE);
    EXPECT(q8(w, s, x, y, 1, 64, 0) == QBD_ERR_SHAPE);
    EXPECT(q8(w, s, x, y, -1, 64, 64) == QBD_ERR_SHAPE);
    EXPECT(q8(w, s, x, y, 1, (int64_t{1} << 31) - (int64_t{1} << 20) + 1, 32) == QBD_ERR_SHAPE);
    EXPECT(q8(w, s, x, y, 1, int64_t{1} << 33, 1 << 10) == QBD_ERR_SHAPE);       // plane >= 2^40
    EXPECT(q8(w, s, x, y, INT64_MAX, INT64_MAX, INT64_MAX - 31) == QBD_ERR_SHAPE);  // no overflow in the checks
    EXPECT(q8(nullptr, s, x, y, 1, 64, 64) == QBD_ERR_NULL);
    EXPECT(q8(w, s, nullptr, y, 1, 64, 64) == QBD_ERR_NULL);
    EXPECT(q8(fake<int8_t>(0, 8), s, x, y, 1, 64, 64) == QBD_ERR_ALIGN);
    EXPECT(q8(w, fake<uint16_t>(1, 1), x, y, 1, 64, 64) == QBD_ERR_ALIGN);
    EXPECT(q8(w, s, fake<float>(2, 4), y, 1, 64, 64) == QBD_ERR_ALIGN);
    EXPECT(q8(w, s, x, fake<float>(3, 2), 1, 64, 64) == QBD_ERR_ALIGN);
    // y overlapping the codes, the scales or x
    EXPECT(q8(w, s, x, reinterpret_cast<float*>(const_cast<int8_t*>(w) + 4096), 1, 64, 4096) == QBD_ERR_ALIAS);
    EXPECT(q8(w, s, x, reinterpret_cast<float*>(const_cast<uint16_t*>(s)), 1, 64, 64) == QBD_ERR_ALIAS);
    EXPECT(q8(w, s, x, const_cast<float*>(x) + 16, 2, 64, 64) == QBD_ERR_ALIAS);
    // y just past x does not overlap
    const int calls = g_last.calls;
    EXPECT(q8(w, s, x, const_cast<float*>(x) + 64, 1, 64, 64) == QBD_OK);
    EXPECT(g_last.calls == calls + 1 && g_last.which == 0 && g_last.M == 1 && g_last.N == 64 && g_last.K == 64);
    // empty calls launch nothing
    EXPECT(q8(w, s, x, y, 0, 64, 64) == QBD_OK && g_last.calls == calls + 1);
    EXPECT(q8(w, s, x, y, 5, 0, 64) == QBD_OK && g_last.calls == calls + 1);
    EXPECT(q8(nullptr, nullptr, nullptr, nullptr, 0, 0, 64) == QBD_OK);
    // the largest accepted sizes reach the launcher
    const int64_t big = (int64_t{1} << 31) - (int64_t{1} << 20);
    auto far = [](int i) { return (uintptr_t{1} << 40) * static_cast<uintptr_t>(i + 1); };
    EXPECT(q8(reinterpret_cast<const int8_t*>(far(0)), reinterpret_cast<const uint16_t*>(far(1)),
              reinterpret_cast<const float*>(far(2)), reinterpret_cast<float*>(far(3)), 1, big, 32) == QBD_OK &&
           g_last.N == big);
    EXPECT(qmv_q4_0_f32(fake<uint8_t>(0), s, x, y, 3, 17, 96, nullptr) == QBD_OK);
    EXPECT(g_last.fmt == qbd::Fmt::Q4 && g_last.mode == qbd::Mode::Plain && g_last.M == 3);
}

void check_from_f32() {
    const int8_t* w = fake<int8_t>(0);
    const uint16_t* s = fake<uint16_t>(1);
    const float* x = fake<float>(2);
    int8_t* xq = fake<int8_t>(3);
    float* xd = fake<float>(4);
    float* y = fake<float>(5);
    auto q8 = [&](const int8_t* w_, const float* x_, int8_t* xq_, float* xd_, float* y_, int64_t M, int64_t N,
                  int64_t K) { return qmm_q8_0_q8act_from_f32(w_, s, x_, xq_, xd_, y_, M, N, K, nullptr); };
    int calls = g_last.calls;
    EXPECT(q8(w, x, xq, xd, y, 1, 4864, 896) == QBD_OK);
    EXPECT(g_last.calls == calls + 1 && g_last.which == 4 && g_last.N == 4864 && g_last.mode == qbd::Mode::Plain);
    EXPECT(q8(w, x, xq, xd, y, 1, 64, 48) == QBD_ERR_SHAPE);
    EXPECT(q8(w, x, nullptr, xd, y, 1, 64, 64) == QBD_ERR_NULL);
    EXPECT(q8(w, x, xq, nullptr, y, 1, 64, 64) == QBD_ERR_NULL);
    EXPECT(q8(w, x, xq, xd, nullptr, 1, 64, 64) == QBD_ERR_NULL);
    EXPECT(q8(w, x, fake<int8_t>(3, 8), xd, y, 1, 64, 64) == QBD_ERR_ALIGN);
    EXPECT(q8(w, x, xq, fake<float>(4, 2), y, 1, 64, 64) == QBD_ERR_ALIGN);
    EXPECT(q8(w, fake<float>(2, 4), xq, xd, y, 1, 64, 64) == QBD_ERR_ALIGN);
    // outputs over an input or over each other
    EXPECT(q8(w, x, reinterpret_cast<int8_t*>(const_cast<float*>(x)), xd, y, 1, 64, 64) == QBD_ERR_ALIAS);
    EXPECT(q8(w, x, xq, reinterpret_cast<float*>(const_cast<int8_t*>(w)) + 4, y, 1, 64, 64) == QBD_ERR_ALIAS);
    EXPECT(q8(w, x, xq, xd, reinterpret_cast<float*>(xq) + 4, 1, 64, 64) == QBD_ERR_ALIAS);
    EXPECT(q8(w, x, xq, reinterpret_cast<float*>(xq + 32), y, 1, 64, 64) == QBD_ERR_ALIAS);
    EXPECT(q8(w, x, xq, xd, xd + 1, 1, 64, 64) == QBD_ERR_ALIAS);
    // xq just past x, xd just past xq: no overlap
    EXPECT(q8(w, x, reinterpret_cast<int8_t*>(const_cast<float*>(x) + 64), xd, y, 1, 64, 64) == QBD_OK);
    EXPECT(q8(w, x, xq, reinterpret_cast<float*>(xq + 64), y, 1, 64, 64) == QBD_OK);
    // M = 0 does nothing; N = 0 still quantizes x
    calls = g_last.calls;
    EXPECT(q8(w, x, xq, xd, y, 0, 64, 64) == QBD_OK && g_last.calls == calls);
    EXPECT(q8(w, nullptr, xq, xd, y, 3, 0, 64) == QBD_ERR_NULL);
    EXPECT(q8(nullptr, x, xq, xd, nullptr, 3, 0, 64) == QBD_OK && g_last.calls == calls + 1 && g_last.which == 1 &&
           g_last.M == 3 && g_last.K == 64);
    // the 4-bit forms
    const uint8_t* w4 = fake<uint8_t>(6);
    EXPECT(qmm_q4_0_q8act_from_f32(w4, s, x, xq, xd, y, 1, 5120, 17408, nullptr) == QBD_OK);
    EXPECT(g_last.which == 4 && g_last.fmt == qbd::Fmt::Q4 && g_last.mode == qbd::Mode::Plain && g_last.K == 17408);
    const uint8_t* u4 = fake<uint8_t>(7);
    const uint16_t* us = fake<uint16_t>(8);
    EXPECT(gate_up_swiglu_q4_q8act_from_f32(w4, s, u4, us, x, xq, xd, y, 1, 17408, 5120, nullptr) == QBD_OK);
    EXPECT(g_last.which == 4 && g_last.mode == qbd::Mode::SwiGLU);
    EXPECT(gate_up_swiglu_q4_q8act_from_f32(w4, s, nullptr, us, x, xq, xd, y, 1, 64, 64, nullptr) == QBD_ERR_NULL);
    EXPECT(gate_up_swiglu_q4_q8act_from_f32(w4, s, u4, us, x, xq, xd,
                                            reinterpret_cast<float*>(const_cast<uint16_t*>(us)), 1, 64, 64,
                                            nullptr) == QBD_ERR_ALIAS);
}

void check_fused() {
    const uint8_t* g = fake<uint8_t>(0);
    const uint16_t* gd = fake<uint16_t>(1);
    const uint8_t* u = fake<uint8_t>(2);
    const uint16_t* ud = fake<uint16_t>(3);
    const float* x = fake<float>(4);
    float* out = fake<float>(5);
    EXPECT(gate_up_swiglu_q4(g, gd, u, ud, x, out, 8, 17408, 5120, nullptr) == QBD_OK);
    EXPECT(g_last.which == 0 && g_last.mode == qbd::Mode::SwiGLU && g_last.fmt == qbd::Fmt::Q4);
    EXPECT(gate_up_swiglu_q4(g, gd, nullptr, ud, x, out, 8, 64, 64, nullptr) == QBD_ERR_NULL);
    EXPECT(gate_up_swiglu_q4(g, gd, u, fake<uint16_t>(3, 1), x, out, 8, 64, 64, nullptr) == QBD_ERR_ALIGN);
    EXPECT(gate_up_swiglu_q4(g, gd, u, ud, x, reinterpret_cast<float*>(const_cast<uint8_t*>(u)) + 8, 1, 64, 64,
                             nullptr) == QBD_ERR_ALIAS);
    EXPECT(gate_up_swiglu_q8_0(fake<int8_t>(0), gd, fake<int8_t>(2), ud, x, out, 1, 4864, 896, nullptr) == QBD_OK);
    EXPECT(g_last.fmt == qbd::Fmt::Q8_0 && g_last.mode == qbd::Mode::SwiGLU);
    const int8_t* xq = fake<int8_t>(6);
    const float* xd = fake<float>(7);
    EXPECT(gate_up_swiglu_q4_q8act(g, gd, u, ud, xq, xd, out, 1024, 17408, 5120, nullptr) == QBD_OK);
    EXPECT(g_last.which == 2 && g_last.mode == qbd::Mode::SwiGLU && g_last.M == 1024);
    EXPECT(gate_up_swiglu_q4_q8act(g, gd, u, ud, xq, nullptr, out, 4, 64, 64, nullptr) == QBD_ERR_NULL);
    EXPECT(gate_up_swiglu_q4_q8act(g, gd, u, ud, xq, fake<float>(7, 2), out, 4, 64, 64, nullptr) == QBD_ERR_ALIGN);
    EXPECT(gate_up_swiglu_q4_q8act(g, gd, u, ud, xq, xd, const_cast<float*>(xd), 4, 64, 64, nullptr) == QBD_ERR_ALIAS);
}

void check_q8act_quantize_swiglu() {
    const int8_t* w = fake<int8_t>(0);
    const uint16_t* s = fake<uint16_t>(1);
    const int8_t* xq = fake<int8_t>(2);
    const float* xd = fake<float>(3);
    float* y = fake<float>(4);
    EXPECT(qmm_q8_0_q8act(w, s, xq, xd, y, 32, 1152, 896, nullptr) == QBD_OK);
    EXPECT(g_last.which == 2 && g_last.fmt == qbd::Fmt::Q8_0 && g_last.N == 1152);
    EXPECT(qmm_q4_0_q8act(fake<uint8_t>(0), s, xq, xd, y, 32, 1152, 896, nullptr) == QBD_OK);
    EXPECT(qmm_q8_0_q8act(w, s, fake<int8_t>(2, 4), xd, y, 1, 64, 64, nullptr) == QBD_ERR_ALIGN);
    EXPECT(qmm_q8_0_q8act(w, s, xq, xd, y, 1, 64, 40, nullptr) == QBD_ERR_SHAPE);

    const float* x = fake<float>(5);
    int8_t* q = fake<int8_t>(6);
    float* d = fake<float>(7);
    EXPECT(quantize_act_q8_0(x, q, d, 4, 896, nullptr) == QBD_OK && g_last.which == 1 && g_last.K == 896);
    EXPECT(quantize_act_q8_0(x, q, d, 4, 900, nullptr) == QBD_ERR_SHAPE);
    EXPECT(quantize_act_q8_0(x, nullptr, d, 4, 896, nullptr) == QBD_ERR_NULL);
    EXPECT(quantize_act_q8_0(x, q, fake<float>(7, 2), 4, 896, nullptr) == QBD_ERR_ALIGN);
    EXPECT(quantize_act_q8_0(x, reinterpret_cast<int8_t*>(const_cast<float*>(x)) + 32, d, 4, 896, nullptr) ==
           QBD_ERR_ALIAS);
    EXPECT(quantize_act_q8_0(x, q, reinterpret_cast<float*>(q + 64), 4, 896, nullptr) == QBD_ERR_ALIAS);

    const float* g = fake<float>(8);
    const float* u = fake<float>(9);
    float* o = fake<float>(10);
    EXPECT(swiglu_f32(g, u, o, 1000, nullptr) == QBD_OK && g_last.which == 3 && g_last.N == 1000);
    EXPECT(swiglu_f32(g, u, o, -1, nullptr) == QBD_ERR_SHAPE);
    EXPECT(swiglu_f32(g, u, const_cast<float*>(u) + 999, 1000, nullptr) == QBD_ERR_ALIAS);
    EXPECT(swiglu_f32(g, u, o, 0, nullptr) == QBD_OK);
}

void check_device() {
    // the device check is cached per device: a non-gfx950 answer would need
    // a fresh process; here the stand-in reports gfx950
    EXPECT(qbd_abi_version() == 1);
    for (int st = -7; st <= 1; ++st) EXPECT(qbd_status_str(st) != nullptr && qbd_status_str(st)[0] != 0);
}

void check_split_helpers() {
    const int64_t N = 3, K = 96, nb = K / 32;
    // Q8_0: 34-byte blocks, little-endian fp16 d first
    std::vector<uint8_t> b34(static_cast<size_t>(N * nb * 34));
    for (size_t i = 0; i < b34.size(); ++i) b34[i] = static_cast<uint8_t>(i * 7 + 3);
    std::vector<int8_t> wq(static_cast<size_t>(N * K));
    std::vector<uint16_t> wd(static_cast<size_t>(N * nb));
    EXPECT(q8_0_split_blocks(b34.data(), wq.data(), wd.data(), N, K) == QBD_OK);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = &b34[static_cast<size_t>((n * nb + b) * 34)];
            EXPECT(wd[static_cast<size_t>(n * nb + b)] == static_cast<uint16_t>(blk[0] | (blk[1] << 8)));
            EXPECT(std::memcmp(&wq[static_cast<size_t>(n * K + b * 32)], blk + 2, 32) == 0);
        }
    // Q4: 18-byte blocks
    std::vector<uint8_t> b18(static_cast<size_t>(N * nb * 18));
    for (size_t i = 0; i < b18.size(); ++i) b18[i] = static_cast<uint8_t>(i * 13 + 1);
    std::vector<uint8_t> wq4(static_cast<size_t>(N * K / 2));
    EXPECT(q4_0_split_blocks(b18.data(), wq4.data(), wd.data(), N, K) == QBD_OK);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = &b18[static_cast<size_t>((n * nb + b) * 18)];
            EXPECT(wd[static_cast<size_t>(n * nb + b)] == static_cast<uint16_t>(blk[0] | (blk[1] << 8)));
            EXPECT(std::memcmp(&wq4[static_cast<size_t>(n * K / 2 + b * 16)], blk + 2, 16) == 0);
        }
    EXPECT(q8_0_split_blocks(b34.data(), wq.data(), wd.data(), N, 33) == QBD_ERR_SHAPE);
    EXPECT(q4_0_split_blocks(nullptr, wq4.data(), wd.data(), N, K) == QBD_ERR_NULL);
    EXPECT(q4_0_split_blocks(nullptr, nullptr, nullptr, 0, K) == QBD_OK);
}

// ---- kernel selection
void check_plans() {
    using namespace qbd::plan;
    const int64_t cus_list[] = {256, 304, 80};
    const int64_t Ms[] = {1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 32, 64, 65, 128, 1024, 8 * 65535, 8 * 65535 + 1};
    const int64_t Ns[] = {1, 17, 896, 1152, 4096, 4104, 4864, 5120, 8200, 17408, 20480, 20481, 24576, 151936};
    const int64_t Ks[] = {32, 96, 896, 1024, 2048, 4096, 4864, 5120, 10240, 16384, 17408, 40960};
    int plans = 0;
    for (int64_t cus : cus_list)
        for (int fi = 0; fi < 2; ++fi) {
            const qbd::Fmt f = fi ? qbd::Fmt::Q4 : qbd::Fmt::Q8_0;
            for (int64_t M : Ms)
                for (int64_t N : Ns)
                    for (int64_t K : Ks) {
                        const F32Plan p = f32_plan(f, M, N, K, cus);
                        ++plans;
                        switch (p.kernel) {
                            case F32Kernel::M1Vgpr:
                                EXPECT(M == 1 && p.sweeps >= 1 && p.sweeps <= max_vgpr_sweeps(f));
                                break;
                            case F32Kernel::M1Sweep:
                                // one wave per sweep: at most 1024 threads, a part slot per wave
                                EXPECT(M == 1 && p.sweeps >= 2 && p.sweeps <= m1_sweep_max_j(f) &&
                                       p.sweeps <= kM1SweepMaxJ && 64 * p.sweeps <= 1024 && N < kM1SweepMaxRows);
                                EXPECT(p.sweeps == m1_sweeps(f, K));
                                break;
                            case F32Kernel::M1Staged:
                                EXPECT(M == 1 && m1_staged_lds_bytes(f, K, resident_rows(N, cus)) <= kLdsBytes);
                                break;
                            case F32Kernel::Mfma:
                                // the budget of two weight matrices, whatever the call
                                EXPECT(M >= 2 && M <= 16);
                                EXPECT(mfma_lds_bytes(kMfmaWaves, p.nt, 2, p.mt, K / 32) <= kLdsBytes);
                                EXPECT(p.nt >= 1 && p.nt <= mfma_max_nt(p.mt) && p.nt <= kMfmaMaxNT);
                                break;
                            case F32Kernel::Resident:
                                EXPECT(M >= 2 && cdiv(M, p.mt) <= kMaxGridY);
                                EXPECT(resident_lds_bytes(p.mt, K, resident_rows(N, cus), false) <= kLdsBytes);
                                break;
                            case F32Kernel::Chunked:
                                EXPECT(M >= 2 && cdiv(M, p.mt) <= kMaxGridY);
                                EXPECT(2 * p.mt * 2 * kPanelKC * 4 <= kLdsBytes);
                                break;
                            case F32Kernel::Generic:
                                EXPECT(M == 1 || cdiv(M, panel_rows(M)) > kMaxGridY);
                                break;
                        }
                        const Q8Plan q = q8act_plan(f, M, N, K, cus);
                        // quantize-and-multiply on the per-row dot4 kernel: M = 1, the
                        // sweeps its registers hold, never where the staged kernel runs
                        if (q8act_m1_qx_per_row(f, M, N, K, cus))
                            EXPECT(M == 1 && m1_sweeps(f, K) <= max_vgpr_sweeps(f) &&
                                   cdiv(N, 4) * K <= kQ8M1QxMaxQuantized &&
                                   (q.kernel == Q8Kernel::Dot4 || q.kernel == Q8Kernel::M1Staged));
                        // quantizing inside the product: only on the staged kernel, in a few rounds
                        if (q8act_m1_quantize_inside(f, M, N, K, cus))
                            EXPECT(q.kernel == Q8Kernel::M1Staged &&
                                   cdiv(K / 8, q8act_m1_waves(N, cus) * kLanes) <= kQ8M1QuantRounds);
                        if (q.kernel == Q8Kernel::M1Staged) {
                            EXPECT(M == 1 && N >= kQ8M1StageMinN &&
                                   q8act_m1_lds_bytes(f, K, resident_rows(N, cus), 2) <= kLdsBytes);
                            for (int64_t nmat = 1; nmat <= 2; ++nmat) {
                                const int64_t S = q8act_m1_group(f, K, nmat);
                                EXPECT(S >= 1 && S <= q8act_m1_max_group(nmat));
                                // groups cover every sweep, the last one is never empty
                                const int64_t J = m1_sweeps(f, K), G = cdiv(J, S);
                                EXPECT(G * S >= J && (G - 1) * S < J);
                            }
                            const int64_t nw = q8act_m1_waves(N, cus);
                            EXPECT(nw == 4 || nw == 8 || nw == 16);
                        } else if (q.kernel == Q8Kernel::Tile16Persist) {
                            const int64_t quads = tile16_quads_per_wave(K);
                            EXPECT(M >= kTile16MinRows && M <= 16 && quads >= kPersistMinQuads &&
                                   quads <= persist_max_quads(f) && cdiv(N, 16) >= 2 * cus && q.waves == 8);
                            // the 4-bit fused form has two matrices; Q8_0 has no fused form here
                            for (int64_t nmat = 1; nmat <= (f == qbd::Fmt::Q4 ? 2 : 1); ++nmat)
                                EXPECT(tile16_lds_bytes(f, quads, nmat, true) <= kLdsBytes);
                            // a wave's slice of a tile is whole 64-lane loads
                            EXPECT((16 * tile16_chunks_per_row(f, quads)) % 64 == 0);
                        } else if (q.kernel == Q8Kernel::Tile16) {
                            const int64_t quads = tile16_quads_per_wave(K);
                            EXPECT(M >= kTile16MinRows && quads >= 1 &&
                                   (f == qbd::Fmt::Q4 ? M <= kTile16MaxRowsQ4 && quads <= kTile16MaxQuadsQ4
                                                      : M <= kTile16MaxRows && quads <= kTile16MaxQuads &&
                                                            (M <= 16 || cdiv(M, 16) * cdiv(N, 16) <= kTile16MaxTiles)));
                            for (int64_t nmat = 1; nmat <= (f == qbd::Fmt::Q4 ? 2 : 1); ++nmat)
                                EXPECT(tile16_lds_bytes(f, quads, nmat, false) <= kLdsBytes);
                            EXPECT((16 * tile16_chunks_per_row(f, quads)) % 64 == 0);
                        }
                        else if (q.kernel == Q8Kernel::PanelStaged) {
                            const int64_t mt = q8act_panel_mt(M);
                            EXPECT(M >= 2 && M <= kPanelStagedMaxRows && N >= kPanelStagedMinN && q.mt == mt &&
                                   mt >= M && (mt == 2 || mt == 4 || mt == 8));
                            for (int64_t nmat = 1; nmat <= 2; ++nmat) {
                                EXPECT(q8act_panel_lds_bytes(f, mt, nmat) <= kLdsBytes);
                                const int64_t rw = q8act_panel_rows_per_wave(nmat);
                                const int64_t rows = q8act_panel_rows(N, nmat, cus);
                                // every row of a workgroup has a wave and a register set
                                EXPECT(rw >= 1 && rows >= 1 && rows <= 16 * rw && cdiv(N, rows) < (int64_t{1} << 31));
                            }
                        } else if (M < kMfmaMinRows) EXPECT(q.kernel == Q8Kernel::Dot4 && q.mt >= 1 && q.mt <= 4);
                        else if (q.kernel == Q8Kernel::SplitK) EXPECT(M <= 64 && (q.waves == 8 || q.waves == 16));
                        else EXPECT(q.kernel == Q8Kernel::Panel);
                    }
        }
    EXPECT(plans > 1000);
    // shapes whose one-matrix budget fits the matrix-core panel but whose
    // two-matrix budget does not: every call takes the VALU panel
    struct S { qbd::Fmt f; int64_t M, N, K; };
    const S shapes[] = {{qbd::Fmt::Q4, 8, 24576, 16384}, {qbd::Fmt::Q8_0, 12, 24576, 16384},
                        {qbd::Fmt::Q4, 8, 8192, 40960}};
    for (const S& s : shapes) {
        EXPECT(f32_plan(s.f, s.M, s.N, s.K, 256).kernel != F32Kernel::Mfma);
        EXPECT(mfma_lds_bytes(kMfmaWaves, mfma_nt(s.M, s.N, 256), 1, mfma_rows(s.M), s.K / 32) <= kLdsBytes);
    }
    // the workloads' kernels
    EXPECT(f32_plan(qbd::Fmt::Q8_0, 1, 151936, 896, 256).kernel == F32Kernel::M1Vgpr);
    EXPECT(f32_plan(qbd::Fmt::Q8_0, 1, 896, 4864, 256).kernel == F32Kernel::M1Sweep);
    EXPECT(q8act_m1_qx_per_row(qbd::Fmt::Q8_0, 1, 1152, 896, 256));
    EXPECT(q8act_m1_qx_per_row(qbd::Fmt::Q8_0, 1, 896, 4864, 256));
    EXPECT(q8act_m1_qx_per_row(qbd::Fmt::Q8_0, 1, 4864, 896, 256));
    EXPECT(!q8act_m1_qx_per_row(qbd::Fmt::Q8_0, 1, 151936, 896, 256));
    EXPECT(!q8act_m1_qx_per_row(qbd::Fmt::Q4, 1, 17408, 5120, 256));
    EXPECT(!q8act_m1_qx_per_row(qbd::Fmt::Q8_0, 1, 300, 8224, 256));
    EXPECT(f32_plan(qbd::Fmt::Q8_0, 1, 1152, 896, 256).kernel == F32Kernel::M1Vgpr);
    EXPECT(f32_plan(qbd::Fmt::Q4, 1, 2000, 16384, 256).kernel == F32Kernel::M1Staged);
    EXPECT(f32_plan(qbd::Fmt::Q4, 8, 17408, 5120, 256).kernel == F32Kernel::Mfma);
    EXPECT(f32_plan(qbd::Fmt::Q4, 1, 17408, 5120, 256).kernel == F32Kernel::M1Staged);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 32, 896, 4864, 256).kernel == Q8Kernel::Tile16);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 32, 4864, 896, 256).kernel == Q8Kernel::SplitK);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 8, 4864, 896, 256).kernel == Q8Kernel::Tile16);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 4, 4864, 896, 256).kernel == Q8Kernel::Tile16);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 2, 4864, 896, 256).kernel == Q8Kernel::PanelStaged);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 3, 17408, 5120, 256).kernel == Q8Kernel::Tile16Persist);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 2, 17408, 5120, 256).kernel == Q8Kernel::PanelStaged);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 5, 4864, 8224, 256).kernel == Q8Kernel::PanelStaged);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 8, 5120, 17408, 256).kernel == Q8Kernel::PanelStaged);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 8, 17408, 5120, 256).kernel == Q8Kernel::Tile16Persist);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 16, 17408, 5120, 256).kernel == Q8Kernel::Tile16Persist);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 8, 17408, 6144, 256).kernel == Q8Kernel::Tile16);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 8, 4096, 5120, 256).kernel == Q8Kernel::Tile16);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 16, 17408, 5120, 256).kernel == Q8Kernel::Tile16Persist);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 8, 151936, 896, 256).kernel == Q8Kernel::Tile16);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 8, 151936, 6144, 256).kernel == Q8Kernel::Tile16Persist);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 8, 151936, 6176, 256).kernel == Q8Kernel::Tile16);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 17, 17408, 5120, 256).kernel != Q8Kernel::Tile16 &&
           q8act_plan(qbd::Fmt::Q4, 17, 17408, 5120, 256).kernel != Q8Kernel::Tile16Persist);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 12, 5120, 17408, 256).kernel == Q8Kernel::Dot4);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 32, 896, 4864, 256).kernel == Q8Kernel::SplitK);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 1024, 17408, 5120, 256).kernel == Q8Kernel::Panel);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 1, 17408, 5120, 256).kernel == Q8Kernel::M1Staged);
    EXPECT(q8act_plan(qbd::Fmt::Q4, 1, 5120, 17408, 256).kernel == Q8Kernel::M1Staged);
    EXPECT(q8act_plan(qbd::Fmt::Q8_0, 1, 896, 896, 256).kernel == Q8Kernel::Dot4);
}

}  // namespace

int main() {
    check_qmv();
    check_fused();
    check_from_f32();
    check_q8act_quantize_swiglu();
    check_device();
    check_split_helpers();
    check_plans();
    if (g_failures) {
        std::fprintf(stderr, "%d checks failed\n", g_failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
