/*
 * qbd.h - C ABI of libqbd, block-quantized decode matmuls for AMD MI355X
 * (gfx950).
 *
 * Formats
 *   Q8_0 weights (native block: 32 signed 8-bit codes q and one fp16 scale d,
 *   weight = d*q; Lumen v0.2.0 release page, "Phase 7.D - Q8-native fused
 *   matmul") are passed as two planes:
 *     wq  int8_t   [N][K]     row n = output feature n, K contiguous
 *     wd  uint16_t [N][K/32]  binary16 bit pattern of block b of row n
 *   Q4 weights (32 four-bit codes q in 0..15 and one fp16 scale d per block,
 *   weight = d*(q-8); the 4-bit gate/up weights of LSE v0.4.16 release page,
 *   "Combined M8 Q4 gate/up execution"):
 *     wq4 uint8_t  [N][K/2]   block b of row n is bytes [16b, 16b+16); byte j
 *                             holds code 32b+j in bits 0-3 and code 32b+16+j
 *                             in bits 4-7
 *     wd  uint16_t [N][K/32]
 *   Q8 activations (per-32-block activation quantization; Lumen v0.4.0
 *   release page, "Phase 7.M - Q8xQ8 AVX2 int dot"):
 *     xq  int8_t   [M][K]     codes, q = round-half-away(x/d)
 *     xd  float    [M][K/32]  d = max|x|/127 (fp32, 0 for an all-zero block)
 *   fp32 activations x [M][K] and outputs y [M][N] are row-major.
 *
 * Conventions (every compute entry point)
 *   - Pointers are device pointers (HBM) unless stated otherwise; the caller
 *     owns every buffer.  Inputs are only read; outputs are fully
 *     overwritten, never accumulated into.  The library allocates no memory
 *     and keeps no workspace: fused entry points write no temporary.
 *   - Arguments are validated on the host before any HIP call.  The call
 *     then enqueues its kernels on `stream` (NULL = the default stream) and
 *     returns without waiting; faults inside a kernel surface at the
 *     caller's next synchronization.
 *   - M = 0 or N = 0 (or n = 0) returns QBD_OK and launches nothing.
 *   - K must be a positive multiple of 32.  M, N, K must be at most
 *     2^31 - 2^20 and every plane below 2^40 bytes (QBD_ERR_SHAPE otherwise).
 *   - Alignment: wq, wq4, x and xq 16 bytes; wd 2 bytes; xd, y, out, g, u
 *     4 bytes.
 *   - No output may overlap any input or another output.
 *   - The current HIP device must be a gfx950 (checked once per device).
 *   - There is no host fallback: what the GPU path cannot do is an error.
 *   - Results are defined per function and never depend on the shape:
 *     (M, N, K) only select the kernel, which may change the fp32
 *     summation order and nothing else.  fp32 outputs match the exact result within
 *     1e-4 * sum|terms| + 1e-6; activation codes, activation scales and the
 *     int32 block dots are exact.  A fused entry point returns the same bits
 *     as its unfused composition at the same M.
 */
#ifndef QBD_H
#define QBD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t of the HIP runtime; NULL selects the default stream. */
typedef struct ihipStream_t* qbd_stream_t;

enum qbd_status {
    QBD_OK = 0,
    QBD_ERR_NULL = -1,   /* a required pointer is NULL */
    QBD_ERR_SHAPE = -2,  /* negative size, K not a positive multiple of 32, too large */
    QBD_ERR_ALIGN = -3,  /* a pointer misses its alignment */
    QBD_ERR_ALIAS = -4,  /* an output overlaps an input or another output */
    QBD_ERR_DEVICE = -5, /* no current HIP device, or it is not a gfx950 */
    QBD_ERR_LAUNCH = -6  /* the kernel launch was rejected by the runtime */
};

/* Static, NUL-terminated description of a status code. */
const char* qbd_status_str(int status);

/* ABI version of this header (incremented on any signature change). */
int qbd_abi_version(void);

/*
 * y[m][n] = sum_k d[n][k/32] * q[n][k] * x[m][k]      (Q8_0 x fp32)
 * The Q8-native decode GEMV without a dequantized weight copy (Lumen v0.2.0
 * release page, "Phase 7.D - Q8-native fused matmul"; M = 1 is the
 * per-token decode shape, "Phase 7.C - 1xN 4-accumulator decode kernel").
 * x [M][K] fp32, y [M][N] fp32.
 */
int qmv_q8_0_f32(const int8_t* wq, const uint16_t* wd, const float* x, float* y,
                 int64_t M, int64_t N, int64_t K, qbd_stream_t stream);

/*
 * Per-32-block Q8 quantization of fp32 activations x [M][K]: for each row m
 * and block b, d = fl32(max|x| / 127) and q = round-half-away(fl32(x / d)),
 * both correctly rounded fp32 divisions; an all-zero block gives d = 0 and
 * q = 0.  Writes xq [M][K] int8 and xd [M][K/32] fp32.  Bit-exact.
 * (Lumen v0.4.0 release page, "Phase 7.M - Q8xQ8 AVX2 int dot":
 * activation quantization pipeline; LSE v0.4.15 release page, "Changes":
 * one activation panel producer shared by several projections.)
 * Non-finite x is outside the contract.
 */
int quantize_act_q8_0(const float* x, int8_t* xq, float* xd,
                      int64_t M, int64_t K, qbd_stream_t stream);

/*
 * y[m][n] = sum_b (d_w[n][b] * d_x[m][b]) * dot[m][n][b],
 * dot[m][n][b] = sum_{i<32} q_w[n][32b+i] * q_x[m][32b+i] formed exactly in
 * int32 before scaling (Q8_0 x Q8 activations; Lumen v0.4.0 release page,
 * "Phase 7.M - Q8xQ8 AVX2 int dot" and "Phase 7.O - 4-accumulator VNNI
 * kernel"; M = 32 is the pp32 prefill shape of Lumen v0.5.0 release page,
 * "Headline").  xq/xd as written by quantize_act_q8_0.
 */
int qmm_q8_0_q8act(const int8_t* wq, const uint16_t* wd, const int8_t* xq, const float* xd,
                   float* y, int64_t M, int64_t N, int64_t K, qbd_stream_t stream);

/*
 * out[m][n] = silu(g[m][n]) * u[m][n], silu(z) = z / (1 + e^-z), where
 * g = x . Wg^T and u = x . Wu^T with Q4 gate/up weights and fp32 x [M][K].
 * One launch, one shared activation panel, no gate temporary, each
 * projection accumulated on its own (LSE v0.4.16 release page, "Combined
 * M8 Q4 gate/up execution").  Bitwise equal to qmv_q4_0_f32 twice followed
 * by swiglu_f32 at the same M.  out [M][N] fp32.
 */
int gate_up_swiglu_q4(const uint8_t* gq, const uint16_t* gd,
                      const uint8_t* uq, const uint16_t* ud,
                      const float* x, float* out,
                      int64_t M, int64_t N, int64_t K, qbd_stream_t stream);

/*
 * The same combined gate/up SwiGLU consumer on Q8_0 gate/up weights
 * (int8 codes [N][K], scales [N][K/32]), as used by the gate and up
 * projections of an 8-bit decode layer: out[m][n] = silu(g[m][n]) * u[m][n]
 * with g = x . Wg^T, u = x . Wu^T, fp32 x [M][K].  One launch, no gate
 * temporary (LSE v0.4.16 release page, "Combined M8 Q4 gate/up
 * execution").  Bitwise equal to qmv_q8_0_f32 twice followed by swiglu_f32
 * at the same M.  out [M][N] fp32.
 */
int gate_up_swiglu_q8_0(const int8_t* gq, const uint16_t* gd, const int8_t* uq,
                        const uint16_t* ud, const float* x, float* out,
                        int64_t M, int64_t N, int64_t K, qbd_stream_t stream);

/*
 * y[m][n] = sum_k d[n][k/32] * (q[n][k] - 8) * x[m][k]   (Q4 x fp32)
 * One projection of the gate/up pair above, as a standalone call.
 */
int qmv_q4_0_f32(const uint8_t* wq4, const uint16_t* wd, const float* x, float* y,
                 int64_t M, int64_t N, int64_t K, qbd_stream_t stream);

/*
 * y[m][n] = sum_b (d_w[n][b] * d_x[m][b]) * dot[m][n][b] with
 * dot = sum_{i<32} (q_w - 8) * q_x exact in int32 (Q4 x Q8 activations; the
 * prefill panels of LSE v0.4.16 release page, "Retained optimizations and
 * compatibility").
 */
int qmm_q4_0_q8act(const uint8_t* wq4, const uint16_t* wd, const int8_t* xq, const float* xd,
                   float* y, int64_t M, int64_t N, int64_t K, qbd_stream_t stream);

/*
 * out = silu(g) * u with g, u the Q4 x Q8-activation products above, fused
 * in one launch.  Bitwise equal to qmm_q4_0_q8act twice followed by
 * swiglu_f32 at the same M.
 */
int gate_up_swiglu_q4_q8act(const uint8_t* gq, const uint16_t* gd,
                            const uint8_t* uq, const uint16_t* ud,
                            const int8_t* xq, const float* xd, float* out,
                            int64_t M, int64_t N, int64_t K, qbd_stream_t stream);

/*
 * Activation quantization and a Q8-activation product in one call, for the
 * matmul that quantizes its own fp32 activations per block before the
 * integer block dots (Lumen v0.4.0 release page, "Phase 7.M - Q8xQ8 AVX2
 * int dot").  x [M][K] fp32 is read; xq [M][K] int8 and xd [M][K/32] fp32
 * (the quantized panel, kept for other consumers of the same activations)
 * and y [M][N] (out for the gate/up form) are written.  Every byte of xq,
 * xd and y equals what quantize_act_q8_0(x, xq, xd) followed by the named
 * product writes; at M = 1 over long weight rows the panel is quantized
 * inside the product's one launch.  Outputs must not overlap any input or
 * each other (QBD_ERR_ALIAS); x, xq 16-byte aligned, xd and y 4-byte
 * aligned.  N = 0 is quantize_act_q8_0 alone: the weight and output
 * pointers are not looked at.
 */
int qmm_q8_0_q8act_from_f32(const int8_t* wq, const uint16_t* wd, const float* x,
                            int8_t* xq, float* xd, float* y,
                            int64_t M, int64_t N, int64_t K, qbd_stream_t stream);
int qmm_q4_0_q8act_from_f32(const uint8_t* wq4, const uint16_t* wd, const float* x,
                            int8_t* xq, float* xd, float* y,
                            int64_t M, int64_t N, int64_t K, qbd_stream_t stream);
int gate_up_swiglu_q4_q8act_from_f32(const uint8_t* gq, const uint16_t* gd,
                                     const uint8_t* uq, const uint16_t* ud,
                                     const float* x, int8_t* xq, float* xd, float* out,
                                     int64_t M, int64_t N, int64_t K, qbd_stream_t stream);

/* out[i] = silu(g[i]) * u[i] for i < n, fp32: the SwiGLU step that follows
 * the two separate gate and up kernels which the combined launch replaces
 * (LSE v0.4.16 release page, "Combined M8 Q4 gate/up execution"); silu as
 * defined above. */
int swiglu_f32(const float* g, const float* u, float* out, int64_t n, qbd_stream_t stream);

/*
 * Host helpers (host memory, no GPU): split interleaved blocks into planes.
 * The blocks stay in their native quantized layout, only split into a codes
 * plane and a scales plane (Lumen v0.2.0 release page, "Phase 7.D": no
 * dequantized weight copy).
 * q8_0_split_blocks: blocks34 holds N*K/32 blocks of 34 bytes (little-endian
 * fp16 d, then 32 int8 codes) in row order; writes wq [N][K], wd [N][K/32].
 * q4_0_split_blocks: blocks18 holds N*K/32 blocks of 18 bytes (fp16 d, then
 * the 16 code bytes in the byte order above); writes wq4 [N][K/2], wd.
 */
int q8_0_split_blocks(const void* blocks34, int8_t* wq, uint16_t* wd, int64_t N, int64_t K);
int q4_0_split_blocks(const void* blocks18, uint8_t* wq4, uint16_t* wd, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* QBD_H */
