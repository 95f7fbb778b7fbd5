"""Block-quantized decode matmuls for AMD MI355X (gfx950).

The compute lives in libqbd.so (HIP kernels behind a C ABI, include/qbd.h);
this package is its thin Python binding plus the seeded input generators.
"""
from .binding import (QbdError, gate_up_swiglu_q4, gate_up_swiglu_q4_q8act,  # noqa: F401
                      gate_up_swiglu_q4_q8act_from_f32, gate_up_swiglu_q8_0, lib, q4_0_split_blocks,
                      q8_0_split_blocks, qmm_q4_0_q8act, qmm_q4_0_q8act_from_f32, qmm_q8_0_q8act,
                      qmm_q8_0_q8act_from_f32, qmv_q4_0_f32, qmv_q8_0_f32, quantize_act_q8_0, status_str,
                      swiglu_f32)
