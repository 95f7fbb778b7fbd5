// Internal launchers of libqbd (host side).  Shapes and pointers have been
// validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "plan.hpp"

namespace qbd {

// y[M][N] = x[M][K] . W^T (Plain), or out = silu(x.Wa^T) * (x.Wb^T) (SwiGLU).
hipError_t launch_qmv_f32(Fmt fmt, Mode mode,
                          const void* wa, const uint16_t* sa,
                          const void* wb, const uint16_t* sb,
                          const float* x, float* y,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream);

// The same product for panels of 2 .. 16 rows on the matrix cores
// (activations split exactly into bf16 parts), for shapes where
// plan::mfma_supported holds; otherwise hipErrorInvalidValue.
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

// Q8_0 or 4-bit weights x Q8 activations for short panels on 16 x 16 int8
// matrix-core tiles (plan::tile16_quads_per_wave(K) <= plan::kTile16MaxQuads),
// one tile per workgroup.
hipError_t launch_qmm_q8_tile16(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa, const void* wb,
                                const uint16_t* sb, const int8_t* xq, const float* xd, float* y, int64_t M,
                                int64_t N, int64_t K, hipStream_t stream);
// The persistent form for one 16-row tile of activations over many weight
// tiles (plan::tile16_persistent).
hipError_t launch_qmm_q8_tile16_persist(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa, const void* wb,
                                        const uint16_t* sb, const int8_t* xq, const float* xd, float* y, int64_t M,
                                        int64_t N, int64_t K, hipStream_t stream);

// The same product on the matrix cores (panels of 16 or more rows).
// quantize_act_q8_0 and launch_qmm_q8act in one call (xq, xd written too)
hipError_t launch_qmm_q8act_from_f32(Fmt fmt, Mode mode, const void* wa, const uint16_t* sa,
                                     const void* wb, const uint16_t* sb, const float* x, int8_t* xq,
                                     float* xd, float* y, int64_t M, int64_t N, int64_t K,
                                     hipStream_t stream);
hipError_t launch_qmm_q8act_mfma(Fmt fmt, Mode mode,
                                 const void* wa, const uint16_t* sa,
                                 const void* wb, const uint16_t* sb,
                                 const int8_t* xq, const float* xd, float* y,
                                 int64_t M, int64_t N, int64_t K, hipStream_t stream);

// CU count of the current device (256 when it cannot be queried).
int device_cus();

// out[i] = silu(g[i]) * u[i].
hipError_t launch_swiglu(const float* g, const float* u, float* out, int64_t n,
                         hipStream_t stream);

}  // namespace qbd
