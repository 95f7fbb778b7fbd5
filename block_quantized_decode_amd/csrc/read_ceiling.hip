// Streaming-read reference for the memory roofline: reads a buffer once and
// folds it into one word per thread, with the load pattern of the weight
// streams it is compared with (16-byte non-temporal loads, consecutive lanes
// on consecutive addresses, one 1024-thread workgroup per compute unit).  Its
// time for B bytes is what one launch can read on this chip, launch and ramp
// included; a product kernel that streams B bytes of weights is measured
// against it.  Not part of the decode path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qbd_ceiling.h"

namespace {

typedef unsigned int u4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 1024;
constexpr int kGroups = 256;

// Thread t folds elements t, t + T, t + 2T, ... (T = all threads) by XOR, so
// the XOR of every output word equals the XOR of every 32-bit word of the
// buffer.
__global__ __launch_bounds__(kThreads) void read_fold(const u4v* __restrict__ p, int64_t n,
                                                        uint32_t* __restrict__ out) {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    uint32_t s = 0;
    int64_t i = tid;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u4v a = __builtin_nontemporal_load(p + i);
        const u4v b = __builtin_nontemporal_load(p + i + stride);
        const u4v c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u4v d = __builtin_nontemporal_load(p + i + 3 * stride);
        s ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
        s ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
    }
    for (; i < n; i += stride) {
        const u4v a = __builtin_nontemporal_load(p + i);
        s ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    out[tid] = s;
}

}  // namespace

extern "C" int64_t qbd_read_ceiling_sink_words(void) { return static_cast<int64_t>(kGroups) * kThreads; }

extern "C" int qbd_read_ceiling(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    if (src == nullptr || sink == nullptr) return -1;
    if (bytes <= 0 || bytes % 16 != 0) return -2;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0) return -3;
    hipLaunchKernelGGL(read_fold, dim3(kGroups), dim3(kThreads), 0, stream, static_cast<const u4v*>(src),
                       bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
