"""bench.py: a multi-GPU request is refused before anything runs; profiler traffic is reported only for the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_entries_follow_the_kernel_sources(tmp_path, monkeypatch):
    """The bench line's `traffic` comes from profiles/traffic.json only while the entry
    was recorded on the current kernel sources; any other hash, or a missing entry,
    gives None (a stale counter run is never reported)."""
    sys.path.insert(0, ROOT)
    import bench

    table = {"eql_fwd4_kernel/c5": {"bytes_per_launch": 123, "source_hash": "current"}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(table))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "current")
    assert bench.traffic_for("eql_fwd4_kernel", "c5") == 123
    assert bench.traffic_for("eql_fwd4_kernel", "c4") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "edited")
    assert bench.traffic_for("eql_fwd4_kernel", "c5") is None


def test_kernel_source_hash_covers_every_source(tmp_path, monkeypatch):
    """Editing any file under csrc/ changes the hash the traffic entries are keyed on."""
    sys.path.insert(0, ROOT)
    import bench

    csrc = tmp_path / "group_circulant_linear_p4_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.h").write_text("int a;")
    (csrc / "b.hip").write_text("int b;")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "b.hip").write_text("int b2;")
    h1 = bench.kernel_source_hash()
    (csrc / "c.h").write_text("")
    h2 = bench.kernel_source_hash()
    assert len({h0, h1, h2}) == 3
