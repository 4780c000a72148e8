"""Host-side pieces of bench.py (no GPU): reading the HBM traffic figure
from a rocprofv3 counter summary, keyed to the kernel sources it measured."""
import bench


def _summary(tmp_path, sha, workload="sweep_s8192_d128", traffic="715306817"):
    p = tmp_path / "counters.md"
    p.write_text(
        "# rocprofv3 HBM byte counters\n\n"
        f"- traffic_bytes_per_launch: `{traffic}`\n"
        f"- kernel_sources_sha256: `{sha}` (fa2_tile.h, fa2_fwd.hip)\n"
        "- library_sha256: `0000`\n"
        f"- workload: `{workload}`\n")
    return str(p)


def test_traffic_read_when_the_sources_match(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", _summary(tmp_path, bench.kernel_source_sha()))
    assert bench.read_traffic("sweep_s8192_d128") == 715306817.0


def test_traffic_null_for_other_sources_or_workload(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", _summary(tmp_path, "f" * 64))
    assert bench.read_traffic("sweep_s8192_d128") is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY",
                        _summary(tmp_path, bench.kernel_source_sha(), workload="other"))
    assert bench.read_traffic("sweep_s8192_d128") is None


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU; --gpus N > 1 exits with a message (before
    touching a device)."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
