// Device helpers shared by the gfx950 kernels of libqbd.
//
// Wave64 reductions use DPP inside 16-lane rows and the gfx950
// v_permlane16_swap / v_permlane32_swap instructions across rows, so no LDS
// is touched.  Every reduction has a fixed summation order, so a kernel that
// calls the same helper on the same partial sums produces the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qbd {

constexpr int kWave = 64;
constexpr int kBlock = 32;  // codes per quantization block

__device__ __forceinline__ float f16_bits_to_f32(uint16_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}

// Per-32-block Q8 activation quantization (Lumen v0.4.0 release page,
// "Phase 7.M - Q8xQ8 AVX2 int dot"): d = max|x| / 127 and
// q = round-half-away(x / d), both divisions correctly rounded fp32 (the
// default fp32 division, no fast math), no flush of subnormals; an all-zero
// block has d = 0 and q = 0.  Every kernel that quantizes activations calls
// these two, so their codes and scales agree bit for bit.
__device__ __forceinline__ float q8_block_scale(float amax) { return amax / 127.0f; }

__device__ __forceinline__ int8_t q8_quantize_one(float v, float d) {
    if (d == 0.f) return 0;
    const float r = v / d;  // correctly rounded
    float q = roundf(r);    // ties away from zero
    q = fminf(fmaxf(q, -127.f), 127.f);
    return static_cast<int8_t>(static_cast<int>(q));
}

// v + v[lane ^ 1], v + v[lane ^ 2], then the 8- and 16-lane mirrors: every
// lane of a 16-lane row ends with the row total.
template <int CTRL>
__device__ __forceinline__ float dpp_shuffle(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_shuffle<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_shuffle<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_shuffle<0x141>(v);  // row_half_mirror
    v += dpp_shuffle<0x140>(v);  // row_mirror
    return v;
}

// permlane32_swap(a, b): a' = [a.lo32, b.lo32], b' = [a.hi32, b.hi32].
// Returns a' + b': lanes 0-31 hold a's half sums, lanes 32-63 b's.
__device__ __forceinline__ float swap32_add(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// permlane16_swap(a, b): a' = [a.r0, b.r0, a.r2, b.r2], b' = [a.r1, b.r1, a.r3, b.r3].
// Returns a' + b'.
__device__ __forceinline__ float swap16_add(float a, float b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reduce R per-lane partials across the wave.  Value r ends in the lane
// returned by reduced_lane<R>(r) (all lanes of that 16-lane row hold it).
template <int R>
__device__ __forceinline__ void wave_reduce(float (&v)[R]);

template <>
__device__ __forceinline__ void wave_reduce<1>(float (&v)[1]) {
    float s = swap32_add(v[0], v[0]);
    s = swap16_add(s, s);
    v[0] = row16_sum(s);
}

template <>
__device__ __forceinline__ void wave_reduce<2>(float (&v)[2]) {
    float s = swap32_add(v[0], v[1]);  // lanes 0-31: v0, 32-63: v1
    s = swap16_add(s, s);
    s = row16_sum(s);
    v[0] = s;
    v[1] = s;
}

template <>
__device__ __forceinline__ void wave_reduce<4>(float (&v)[4]) {
    float p = swap32_add(v[0], v[1]);  // lanes 0-31: v0, 32-63: v1
    float q = swap32_add(v[2], v[3]);  // lanes 0-31: v2, 32-63: v3
    float s = swap16_add(p, q);        // rows: v0, v2, v1, v3
    s = row16_sum(s);
    v[0] = s; v[1] = s; v[2] = s; v[3] = s;
}

// Reduce N per-lane partials (N a multiple of 4) across the wave with the
// same per-value tree as wave_reduce<1>: lane l + 32 onto l, then l + 16
// onto l, then the 16-lane row sum.  Value v ends in 16-lane row
// {0, 2, 1, 3}[v % 4] of register v / 4 (lanes 0, 32, 16, 48 hold values
// 4i, 4i + 1, 4i + 2, 4i + 3 of v[i]).
template <int N>
__device__ __forceinline__ void wave_reduce_many(const float (&in)[N], float (&out)[N / 4]) {
    static_assert(N % 4 == 0, "multiple of four values");
    float p[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) p[i] = swap32_add(in[2 * i], in[2 * i + 1]);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) out[i] = row16_sum(swap16_add(p[2 * i], p[2 * i + 1]));
}

// Lane that holds value v % 4 of a wave_reduce_many result register.
__host__ __device__ constexpr int many_lane(int v4) {
    return v4 == 0 ? 0 : (v4 == 1 ? 32 : (v4 == 2 ? 16 : 48));
}

template <int R>
__host__ __device__ constexpr int reduced_lane(int r);

template <> __host__ __device__ constexpr int reduced_lane<1>(int) { return 0; }
template <> __host__ __device__ constexpr int reduced_lane<2>(int r) { return r == 0 ? 0 : 32; }
template <> __host__ __device__ constexpr int reduced_lane<4>(int r) {
    return r == 0 ? 0 : (r == 1 ? 32 : (r == 2 ? 16 : 48));
}

// Signed byte i (0..3) of a 32-bit word as float (exact).
template <int I>
__device__ __forceinline__ float sbyte_f32(uint32_t w) {
    return static_cast<float>(static_cast<int8_t>((w >> (8 * I)) & 0xFF));
}

// 4-bit codes as signed bytes 16 (q - 8).  Flipping bit 3 of a nibble
// turns the code q into the two's-complement 4-bit number q - 8; with the
// nibble at the top of its byte the byte reads 16 (q - 8).  One shift and
// two mask/xor steps per 4 bytes, then one signed-byte convert per code.
// The factor 16 is exact and is taken back out of the block scale (q4_scale).
__device__ __forceinline__ uint32_t q4x16_lo(uint32_t w) { return ((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u; }
__device__ __forceinline__ uint32_t q4x16_hi(uint32_t w) { return (w & 0xF0F0F0F0u) ^ 0x80808080u; }

// Block scale of a 4-bit block paired with codes from q4x16_*: d / 16,
// exact in fp32 (d is a binary16 value, so d / 16 >= 2^-28 stays normal).
// A power-of-two factor commutes with fp32 rounding wherever no value is
// subnormal, so d/16 * (sum of 16 (q - 8) x) then rounds exactly as
// d * (sum of (q - 8) x) would; with subnormal terms the scaled sums keep
// more bits, never fewer.
__device__ __forceinline__ float q4_scale(uint16_t bits) { return f16_bits_to_f32(bits) * 0.0625f; }

// silu(z) = z / (1 + e^-z), fp32, correctly rounded division.
__device__ __forceinline__ float silu_f32(float z) {
    return z / (1.0f + expf(-z));
}

__device__ __forceinline__ float swiglu_f32(float g, float u) {
    return silu_f32(g) * u;
}

}  // namespace qbd
