"""bench.py's command line on a machine without a GPU: more than one GPU is
refused with a message before anything touches torch or the library."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line


def test_launcher_world_size_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = _run(env=env)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr


def test_help_lists_the_sections():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--secondary", "--extra", "--denoise-steps", "--denoise-reuse",
                 "--sparse", "--w8a8"):
        assert flag in r.stdout


def test_roofline_traffic_only_for_the_source_it_was_measured_on(monkeypatch):
    import hashlib
    import importlib
    import sys as _sys
    _sys.path.insert(0, ROOT)
    bench = importlib.import_module("bench")
    with open(os.path.join(ROOT, "joint_video_audio_h3_amd", "csrc", "attention.hip"), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    monkeypatch.setattr(bench, "TRAFFIC_BYTES", {("w", "attention"): (1.5e9, sha)})
    assert bench.measured_traffic("w", "attention") == 1.5e9
    monkeypatch.setattr(bench, "TRAFFIC_BYTES", {("w", "attention"): (1.5e9, "0" * 16)})
    assert bench.measured_traffic("w", "attention") is None
    assert bench.measured_traffic("other", "attention") is None
