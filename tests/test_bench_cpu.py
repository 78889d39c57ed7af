"""bench.py pieces that need no GPU: the one-GPU refusal and the rule that
reports HBM traffic only from counters taken on the current kernel source."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write_counters(root, name, sha, traffic):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", "%s_counters.md" % name), "w") as f:
        f.write("# counters\n\ntraffic_bytes_per_launch: %d\nkernel_source_sha256_16: %s\n"
                % (traffic, sha))


def test_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    assert len(sha) == 16 and int(sha, 16) >= 0
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: sha)
    assert bench.committed_traffic("w") is None                  # no counters file
    _write_counters(str(tmp_path), "w", sha, 74148387)
    assert bench.committed_traffic("w") == 74148387.0
    other = "%016x" % (int(sha, 16) ^ 1)
    _write_counters(str(tmp_path), "w", other, 74148387)
    assert bench.committed_traffic("w") is None                  # stale counters


def test_kernel_source_hash_follows_the_sources(tmp_path, monkeypatch):
    """The hash covers every file of the kernel sources, by name and content."""
    src = tmp_path / "block_quantized_decode_q4_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "a.hip").write_text("x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_hash()
    (src / "a.hip").write_text("y")
    h2 = bench.kernel_source_hash()
    (src / "b.h").write_text("")
    h3 = bench.kernel_source_hash()
    (src / "b.h").rename(src / "c.h")
    h4 = bench.kernel_source_hash()
    assert len({h1, h2, h3, h4}) == 4


def test_every_kernel_has_a_dtype_and_name():
    """bench.py names the arithmetic of whatever kernel the plan picks."""
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                  "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert set(mod.KERNEL_DTYPE) == set(range(1, 8)) == set(mod.KERNEL_NAMES)
