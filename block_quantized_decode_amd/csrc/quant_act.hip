// Per-32-block Q8 activation quantization on gfx950.
//
// The activation quantization that feeds the Q8 x Q8 matmul (Lumen v0.4.0
// release page, "Phase 7.M - Q8xQ8 AVX2 int dot") and the shared activation
// panel producer (LSE v0.4.15 release page, "Changes").  Per row and block:
// d = max|x| / 127 and q = round-half-away(x / d), both divisions correctly
// rounded fp32 (hipcc's default fp32 division), no flush of subnormals; an
// all-zero block gets d = 0 and q = 0.
//
// Four lanes own one block, eight consecutive floats each (two 16-byte
// loads); the block maximum is two DPP steps inside the lane quad.
#include "device_common.hpp"
#include "launch.hpp"

namespace qbd {
namespace {

__global__ __launch_bounds__(256) void quantize_q8_kernel(
    const float* __restrict__ x, int8_t* __restrict__ xq, float* __restrict__ xd,
    int64_t total_groups) {
    // group g = 8 consecutive floats; groups 4b..4b+3 form block b.
    const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool live = g < total_groups;
    float v[8];
    if (live) {
        const float4 a = *reinterpret_cast<const float4*>(x + 8 * g);
        const float4 b = *reinterpret_cast<const float4*>(x + 8 * g + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // quads are aligned to blocks because blocks are 4 groups and the
    // launch covers whole blocks from group 0
    amax = fmaxf(amax, dpp_shuffle<0xB1>(amax));
    amax = fmaxf(amax, dpp_shuffle<0x4E>(amax));
    const float d = q8_block_scale(amax);
    if (!live) return;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo |= (static_cast<uint32_t>(static_cast<uint8_t>(q8_quantize_one(v[i], d)))) << (8 * i);
        hi |= (static_cast<uint32_t>(static_cast<uint8_t>(q8_quantize_one(v[4 + i], d)))) << (8 * i);
    }
    *reinterpret_cast<uint2*>(xq + 8 * g) = make_uint2(lo, hi);
    if ((g & 3) == 0) xd[g >> 2] = d;
}

}  // namespace

hipError_t launch_quantize_q8(const float* x, int8_t* xq, float* xd, int64_t M, int64_t K,
                              hipStream_t stream) {
    const int64_t groups = M * K / 8;
    const int64_t blocks = (groups + 255) / 256;
    hipLaunchKernelGGL(quantize_q8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       x, xq, xd, groups);
    return hipGetLastError();
}

}  // namespace qbd
