"""Every kernel instantiation of libqbd compiles without scratch (register
spills or stack), from hipcc's kernel-resource-usage remarks.  CPU only:
hipcc cross-compiles for gfx950 without a GPU."""
import shutil

import pytest

from block_quantized_decode_amd import build


def test_no_kernel_uses_scratch():
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    if shutil.which("c++filt") is None:
        pytest.skip("c++filt not found")
    rows = build.resource_usage()
    families = {build._short_name(r["kernel"]).split("<")[0] for r in rows}
    for fam in ("qmv_f32_m1", "qmv_f32_m1_pipe", "qmv_f32_m1_staged", "qmv_f32_m1_sweep", "qmv_f32_mfma", "qmm_mfma_dma",
                "qmm_mfma_kernel", "qmm_mfma_splitk", "qmm_q8act_generic", "quantize_q8_kernel"):
        assert fam in families, fam
    spills = [(r["kernel"], r["scratch"]) for r in rows if r.get("scratch", 0)]
    assert not spills, spills
    assert all(r.get("vgpr", 0) + r.get("agpr", 0) <= 512 for r in rows)
