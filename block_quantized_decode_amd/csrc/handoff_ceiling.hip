// Reference kernels for the cost of a dependent step on the device (a
// measurement aid, not part of the decode path).
//
// A decode token is a chain of dependent products: each reads the previous
// one's output vector.  The chain can be cut into kernel launches (one per
// product, replayed from a HIP graph) or run inside one persistent grid that
// hands each output vector to every workgroup before the next product
// starts.  qbd_empty_launch measures the first form's cost per step (a
// launch that does nothing), qbd_grid_handoff the second's: one workgroup
// per CU, and per phase every workgroup writes its share of a 4 KB vector,
// arrives, waits for all others, then reads the whole vector back and
// counts the values that are not the ones just written.
//
// The handoff uses agent-scope relaxed atomics for the vector and for the
// arrival words, so no L2 write-back or invalidation is needed; the arrive
// follows a wait for the vector's stores.  Three arrival forms:
//   0  one counter, one atomic add per workgroup and phase;
//   1  16 counters on separate 256-byte lines (workgroup g adds to g % 16),
//      each waiter polls all 16;
//   2  one word per workgroup, set to the phase number by a plain store,
//      each waiter polls all of them.
// Every wait is bounded: a workgroup that polls kPollLimit times without
// seeing all arrivals sets the timeout word and leaves, so every other
// workgroup then times out too and the grid ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qbd_ceiling.h"

namespace {

constexpr int kGroups = 256;
constexpr int kVec = 1024;            // floats handed over per phase
constexpr int kArriveWords = 1024;    // counters or per-workgroup words
constexpr int kDataWord = kArriveWords;
constexpr int kErrWord = kArriveWords + 2 * kVec;  // [0] timeout, [1] wrong values
constexpr int64_t kWorkWords = kErrWord + 64;
constexpr unsigned kPollLimit = 400000;

__device__ __forceinline__ unsigned load_agent(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MODE>
__global__ __launch_bounds__(64) void grid_handoff(unsigned* __restrict__ work, int phases) {
    const int g = blockIdx.x, ng = gridDim.x, lane = threadIdx.x;
    const int per = kVec / ng;
    unsigned* arrive = work;
    float* data = reinterpret_cast<float*>(work + kDataWord);
    unsigned* err = work + kErrWord;
    for (int p = 0; p < phases; ++p) {
        float* buf = data + (p & 1) * kVec;  // two buffers: phase p + 2 reuses p's
        if (lane < per)
            __hip_atomic_store(&buf[g * per + lane], static_cast<float>((g * per + lane) * 7 + p),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);  // the vector's stores are acknowledged
        __syncthreads();
        if (lane == 0) {
            if (MODE == 0) __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (MODE == 1)
                __hip_atomic_fetch_add(arrive + 64 * (g & 15), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (MODE == 2) __hip_atomic_store(arrive + g, unsigned(p + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        bool timed_out = false;
        for (unsigned polls = 0;; ++polls) {
            bool all;
            if (MODE == 0) {
                all = __shfl(load_agent(arrive), 0) >= unsigned(p + 1) * unsigned(ng);
            } else if (MODE == 1) {
                all = __all(load_agent(arrive + 64 * (lane & 15)) >= unsigned(p + 1) * unsigned(ng / 16));
            } else {
                bool ok = true;
                for (int i = lane; i < ng; i += 64) ok &= load_agent(arrive + i) >= unsigned(p + 1);
                all = __all(ok);
            }
            if (all) break;
            if (polls >= kPollLimit) { timed_out = true; break; }
        }
        if (timed_out) {  // uniform across the wave
            if (lane == 0) atomicOr(err, 1u);
            return;
        }
        unsigned wrong = 0;
        for (int i = lane; i < kVec; i += 64) {
            const float r = __hip_atomic_load(&buf[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wrong += r != static_cast<float>(i * 7 + p);
        }
        if (wrong) atomicAdd(err + 1, wrong);
    }
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" int64_t qbd_grid_handoff_work_words(void) { return kWorkWords; }

extern "C" int qbd_grid_handoff(int mode, int phases, uint32_t* work, hipStream_t stream) {
    if (work == nullptr) return -1;
    if (mode < 0 || mode > 2 || phases < 0 || phases > (1 << 20)) return -2;
    if (reinterpret_cast<uintptr_t>(work) % 256 != 0) return -3;
    // arrival words and the error words start at zero (the vector need not)
    if (hipMemsetAsync(work, 0, kArriveWords * 4, stream) != hipSuccess ||
        hipMemsetAsync(work + kErrWord, 0, 64 * 4, stream) != hipSuccess)
        return -6;
    void* args[] = {&work, &phases};
    const void* fn = mode == 0 ? reinterpret_cast<const void*>(grid_handoff<0>)
                   : mode == 1 ? reinterpret_cast<const void*>(grid_handoff<1>)
                               : reinterpret_cast<const void*>(grid_handoff<2>);
    // a cooperative launch: the runtime refuses it unless every workgroup is
    // resident at once, which the waits rely on
    if (hipLaunchCooperativeKernel(fn, dim3(kGroups), dim3(64), args, 0, stream) != hipSuccess) return -6;
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int qbd_empty_launch(hipStream_t stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
