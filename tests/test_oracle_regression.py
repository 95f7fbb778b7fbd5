"""The oracle reproduces its frozen small outputs bit for bit."""
import json
import os

import numpy as np

from golden.make_oracle_regression import encode, inputs, outputs

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_regression.json")


def test_oracle_regression():
    with open(PATH) as f:
        want = json.load(f)["outputs"]
    got = {k: encode(v) for k, v in outputs(inputs()).items()}
    assert sorted(got) == sorted(want)
    for k in want:
        assert got[k] == want[k], k
