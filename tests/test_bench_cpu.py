"""bench.py's contract pieces that run without a GPU: the one-GPU guard and
the HBM-traffic record reader."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_is_used_only_with_the_sources_it_was_taken_with(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    rec = tmp_path / "profiles" / "w_hbm_traffic.txt"
    body = "# comment: 1\nkernels: k<1>\nhbm_bytes_per_call: 123456789\n"
    rec.write_text(f"kernel_sources_sha256: {bench.kernel_digest('v1')}\n" + body)
    assert bench.hbm_traffic("v1", "w") == 123456789
    # the same record read for a workload whose kernels differ: void
    assert bench.hbm_traffic("decode", "w") is None
    rec.write_text("kernel_sources_sha256: 0\n" + body)
    assert bench.hbm_traffic("v1", "w") is None
    assert bench.hbm_traffic("v1", "absent") is None


def test_every_leg_has_its_sources():
    for leg in bench.LEGS:
        assert leg in bench.SOURCES
        for name in bench.SOURCES[leg]:
            assert os.path.exists(os.path.join(bench.CSRC, name)), name
