"""Host-side logic of bench.py, no GPU: the multi-GPU refusal and the rule
that HBM traffic is reported only while the GEMV source still matches the
one the committed counter profile was taken with."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _profile_sha():
    with open(bench.TRAFFIC_PROFILE) as f:
        for ln in f:
            if ln.startswith("kernel_source_sha256_16="):
                return ln.split("=", 1)[1].strip()
    return None


def test_traffic_read_while_source_matches(tmp_path, monkeypatch):
    # the committed profile against a copy of the source it was taken with
    # stands in for an unchanged kernel
    sha = _profile_sha()
    assert sha is not None
    if bench.source_sha(bench.GEMV_SOURCE) == sha:
        t = bench.traffic_from_profile(None)
        assert isinstance(t, int)
        # a weight stream read once: within a few percent above the
        # 144,643,072 algorithmic bytes of the 151936 x 896 launch
        assert 144_643_072 <= t <= 1.05 * 144_643_072
    else:
        # the kernel source changed since the counters were taken
        assert bench.traffic_from_profile(None) is None
        monkeypatch.setattr(bench, "source_sha", lambda path: sha)
        t = bench.traffic_from_profile(None)
        assert isinstance(t, int) and 144_643_072 <= t <= 1.05 * 144_643_072


def test_traffic_dropped_once_source_differs(tmp_path, monkeypatch):
    other = tmp_path / "qmv_f32.hip"
    with open(bench.GEMV_SOURCE, "rb") as f:
        other.write_bytes(f.read() + b"\n// changed\n")
    monkeypatch.setattr(bench, "GEMV_SOURCE", str(other))
    assert bench.traffic_from_profile(None) is None


def test_traffic_missing_profile(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "absent.txt"))
    assert bench.traffic_from_profile(None) is None


def test_pct_us_is_p10_p50_p90_in_microseconds():
    # linear interpolation between order statistics: 1.4, 3.0 and 4.6 ms
    assert bench.pct_us([3.0, 1.0, 2.0, 5.0, 4.0]) == [1400.0, 3000.0, 4600.0]
