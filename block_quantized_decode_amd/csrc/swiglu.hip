// out = silu(g) * u elementwise, the unfused half of the gate/up SwiGLU
// consumer (LSE v0.4.16 release page, "Combined M8 Q4 gate/up execution").
// It calls the same device silu as the fused kernels, so composing two
// projections with it reproduces the fused output bit for bit.
#include "device_common.hpp"
#include "launch.hpp"

namespace qbd {
namespace {

__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ g,
                                                     const float* __restrict__ u,
                                                     float* __restrict__ out, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = swiglu_f32(g[i], u[i]);
}

}  // namespace

hipError_t launch_swiglu(const float* g, const float* u, float* out, int64_t n, hipStream_t stream) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(swiglu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       g, u, out, n);
    return hipGetLastError();
}

}  // namespace qbd
