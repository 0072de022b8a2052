"""bench.py's host-side contract that needs no GPU: more than one GPU is refused with a
message and exit status 2, before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_is_used_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    prof = tmp_path / "traffic.md"
    good = bench.source_hash(str(src))
    prof.write_text(f"# summary\n\n- hbm_bytes_per_launch: 1.25e+10\n- attention.hip sha256[:16]: {good}\n")
    monkeypatch.setattr(bench, "ATTN_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.read_traffic() == 1.25e10
    src.write_text("// kernel source, changed\n")
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.read_traffic() is None
