// Internal launchers of libqbd (host side).  Shapes and pointers have been
// validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qbd {

enum class Fmt : int { Q8_0 = 0, Q4 = 1 };
enum class Mode : int { Plain = 0, SwiGLU = 1 };

// y[M][N] = x[M][K] . W^T (Plain), or out = silu(x.Wa^T) * (x.Wb^T) (SwiGLU).
hipError_t launch_qmv_f32(Fmt fmt, Mode mode,
                          const void* wa, const uint16_t* sa,
                          const void* wb, const uint16_t* sb,
                          const float* x, float* y,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream);

// The same product for panels of 2 .. 16 rows on the matrix cores
// (activations split exactly into bf16 parts).  Supported when there is at
// least one 16-row tile per CU and the workgroup's scale rows and weight
// stages fit in LDS; otherwise hipErrorInvalidValue.
bool qmv_f32_mfma_supported(Fmt fmt, Mode mode, int64_t M, int64_t N, int64_t K);
// Whether the matrix-core panel is the faster choice for a supported shape.
bool qmv_f32_mfma_preferred(Fmt fmt, int64_t M, int64_t N);
hipError_t launch_qmv_f32_mfma(Fmt fmt, Mode mode,
                               const void* wa, const uint16_t* sa,
                               const void* wb, const uint16_t* sb,
                               const float* x, float* y,
                               int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Per-32 Q8 activation quantization of x[M][K].
hipError_t launch_quantize_q8(const float* x, int8_t* xq, float* xd,
                              int64_t M, int64_t K, hipStream_t stream);

// Weights x Q8 activations: exact int32 block dots, fp32 scaled sum.
hipError_t launch_qmm_q8act(Fmt fmt, Mode mode,
                            const void* wa, const uint16_t* sa,
                            const void* wb, const uint16_t* sb,
                            const int8_t* xq, const float* xd, float* y,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);

// The same product on the matrix cores (panels of 16 or more rows).
hipError_t launch_qmm_q8act_mfma(Fmt fmt, Mode mode,
                                 const void* wa, const uint16_t* sa,
                                 const void* wb, const uint16_t* sb,
                                 const int8_t* xq, const float* xd, float* y,
                                 int64_t M, int64_t N, int64_t K, hipStream_t stream);

// out[i] = silu(g[i]) * u[i].
hipError_t launch_swiglu(const float* g, const float* u, float* out, int64_t n,
                         hipStream_t stream);

}  // namespace qbd
