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

#include <mutex>

#include "qbd_ceiling.h"

namespace {

constexpr int kGroups = 256;
constexpr int kVec = 1024;            // floats handed over per phase
constexpr int kArriveWords = 1024;    // counters or per-workgroup words
constexpr int kDataWord = kArriveWords;
constexpr int kErrWord = kArriveWords + 2 * kVec;  // [0] timeout, [1] wrong values
constexpr int64_t kWorkWords = kErrWord + 64;
constexpr int64_t kResultWords = 64 + kVec;     // error words, then the last vector
constexpr unsigned kPollLimit = 400000;
constexpr int kMaxDevices = 128;

__device__ __forceinline__ unsigned load_agent(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// arrive: kArriveWords words, zero at the start; data: two kVec-float
// vectors; err: the timeout and wrong-value words, zero at the start.
template <int MODE>
__global__ __launch_bounds__(64) void grid_handoff(unsigned* __restrict__ arrive, float* __restrict__ data,
                                                    unsigned* __restrict__ err, int phases) {
    const int g = blockIdx.x, ng = gridDim.x, lane = threadIdx.x;
    const int per = kVec / ng;
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

// Zero the arrival words and the error words (a kernel, not a memset node,
// so that the clearing is an ordinary launch on the stream).
__global__ __launch_bounds__(256) void clear_words(unsigned* __restrict__ arrive, unsigned* __restrict__ err) {
    for (int i = threadIdx.x; i < kArriveWords; i += 256) arrive[i] = 0u;
    if (threadIdx.x < 64) err[threadIdx.x] = 0u;
}

// Copy the vector of the last phase out to out[0 .. kVec) (one workgroup).
__global__ __launch_bounds__(256) void copy_vector(const float* __restrict__ data, int phases, float* __restrict__ out) {
    const float* last = data + ((phases - 1) & 1) * kVec;
    for (int i = threadIdx.x; i < kVec; i += 256) out[i] = last[i];
}

__global__ void empty_kernel() {}

// The work buffer of the allocation-free entry point: one per GPU, held by
// the library until the process ends, at the address hipGetSymbolAddress
// gives on that device (the host-side name is only a stand-in).
static __device__ __align__(256) uint32_t scratch[kWorkWords];

int check_args(int mode, int phases) {
    return mode < 0 || mode > 2 || phases < 0 || phases > (1 << 20) ? -2 : 0;
}

int run_handoff(int mode, int phases, unsigned* arrive, float* data, unsigned* err, hipStream_t stream) {
    hipLaunchKernelGGL(clear_words, dim3(1), dim3(256), 0, stream, arrive, err);
    if (hipGetLastError() != hipSuccess) return -6;
    void* args[] = {&arrive, &data, &err, &phases};
    const void* fn = mode == 0 ? reinterpret_cast<const void*>(grid_handoff<0>)
                   : mode == 1 ? reinterpret_cast<const void*>(grid_handoff<1>)
                               : reinterpret_cast<const void*>(grid_handoff<2>);
    // a cooperative launch: the runtime refuses it unless every workgroup is
    // resident at once, which the waits rely on
    if (hipLaunchCooperativeKernel(fn, dim3(kGroups), dim3(64), args, 0, stream) != hipSuccess) return -6;
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
uint32_t* scratch_ptr() {
    static std::mutex mu;
    static uint32_t* ptrs[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        ptrs[dev] = static_cast<uint32_t*>(p);
    }
    return ptrs[dev];
}

}  // namespace

extern "C" int64_t qbd_grid_handoff_work_words(void) { return kWorkWords; }

extern "C" int qbd_grid_handoff(int mode, int phases, uint32_t* work, hipStream_t stream) {
    if (work == nullptr) return -1;
    if (check_args(mode, phases) != 0) return -2;
    if (reinterpret_cast<uintptr_t>(work) % 256 != 0) return -3;
    return run_handoff(mode, phases, work, reinterpret_cast<float*>(work + kDataWord), work + kErrWord, stream);
}

extern "C" int64_t qbd_grid_handoff_noalloc_result_words(void) { return kResultWords; }

extern "C" int qbd_grid_handoff_noalloc(int mode, int phases, uint32_t* result, hipStream_t stream) {
    if (result == nullptr) return -1;
    if (check_args(mode, phases) != 0) return -2;
    if (reinterpret_cast<uintptr_t>(result) % 4 != 0) return -3;
    uint32_t* const work = scratch_ptr();
    if (work == nullptr) return -5;
    const int st = run_handoff(mode, phases, work, reinterpret_cast<float*>(work + kDataWord), result, stream);
    if (st != 0 || phases == 0) return st;
    hipLaunchKernelGGL(copy_vector, dim3(1), dim3(256), 0, stream, reinterpret_cast<const float*>(work + kDataWord),
                       phases, reinterpret_cast<float*>(result + 64));
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int qbd_empty_launch(hipStream_t stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
