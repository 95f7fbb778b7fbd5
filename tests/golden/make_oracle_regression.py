"""Write oracle_regression.json: small oracle outputs frozen as fp32 bits.

Calls only oracle/.  Inputs are drawn here from a fixed numpy seed.  Rerun
(python tests/golden/make_oracle_regression.py) only when a change to the
oracle's arithmetic is justified by a reading of the pages.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def inputs():
    rng = np.random.default_rng(20240601)
    m, n, k = 3, 5, 96
    return dict(
        wq=rng.integers(-128, 128, size=(n, k), dtype=np.int8),
        wd=rng.uniform(0.001, 0.02, size=(n, k // 32)).astype(np.float16).view(np.uint16),
        gq=rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8),
        gd=rng.uniform(0.002, 0.03, size=(n, k // 32)).astype(np.float16).view(np.uint16),
        uq=rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8),
        ud=rng.uniform(0.002, 0.03, size=(n, k // 32)).astype(np.float16).view(np.uint16),
        x=(rng.standard_normal((m, k)) * np.where(rng.random((m, k)) < 0.05, 20, 1)).astype(np.float32),
    )


def outputs(t):
    xq, xd = oracle.quantize_act_q8_0(t["x"])
    return {
        "qmv_q8_0_f32": oracle.qmv_q8_0_f32(t["wq"], t["wd"], t["x"])[0],
        "qmv_q4_0_f32": oracle.qmv_q4_0_f32(t["gq"], t["gd"], t["x"])[0],
        "quantize_q": xq,
        "quantize_d": xd,
        "qmm_q8_0_q8act": oracle.qmm_q8_0_q8act(t["wq"], t["wd"], xq, xd)[0],
        "qmm_q4_0_q8act": oracle.qmm_q4_0_q8act(t["gq"], t["gd"], xq, xd)[0],
        "gate_up_swiglu_q4": oracle.gate_up_swiglu_q4(t["gq"], t["gd"], t["uq"], t["ud"], t["x"])["out32"],
        "gate_up_swiglu_q4_q8act": oracle.gate_up_swiglu_q4_q8act(
            t["gq"], t["gd"], t["uq"], t["ud"], xq, xd)["out32"],
    }


def encode(a):
    a = np.asarray(a)
    if a.dtype == np.float32:
        return {"dtype": "f32bits", "shape": list(a.shape),
                "data": [f"{v:08x}" for v in a.view(np.uint32).ravel().tolist()]}
    return {"dtype": str(a.dtype), "shape": list(a.shape), "data": a.ravel().tolist()}


if __name__ == "__main__":
    out = {k: encode(v) for k, v in outputs(inputs()).items()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as f:
        json.dump({"source": "written by make_oracle_regression.py (oracle only)", "outputs": out}, f)
    print("wrote", path)
