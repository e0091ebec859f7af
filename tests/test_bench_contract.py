"""CPU checks of bench.py's contract that need no GPU: the multi-GPU refusal,
and that the HBM-traffic figure it reports belongs to the GEMM source in the
tree (the figure comes from rocprofv3 counters taken on that source, recorded
in profiles/)."""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (main() only runs as a script)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_figure_matches_gemm_source():
    assert bench.GEMM_TRAFFIC["source_sha1"] == bench._gemm_source_sha1(), (
        "gemm.hip changed since the FETCH_SIZE/WRITE_SIZE profile: re-take it and update "
        "GEMM_TRAFFIC")
    assert 0.3e9 < bench.GEMM_TRAFFIC["bytes_per_launch"] < 5e9


def test_profiles_name_their_commands():
    files = glob.glob(os.path.join(ROOT, "profiles", "*.md"))
    assert files
    for f in files:
        text = open(f).read()
        assert "rocprofv3" in text and "bench.py" in text, f
