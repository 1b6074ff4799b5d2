"""The CPU ABI tests again, against the library with its host code built under
AddressSanitizer and UndefinedBehaviorSanitizer (g++; the kernels are the
ordinary hipcc objects and are never launched here).  Any out-of-bounds access,
use after free or undefined behaviour in the argument checks, workspace carving
or error paths of the C ABI fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

from joint_video_audio_h3_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    gcc = shutil.which("gcc")
    if gcc is None:
        return None
    p = subprocess.run([gcc, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(900)
def test_abi_under_host_sanitizers():
    asan = _runtime("libasan.so")
    if shutil.which("g++") is None or asan is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("g++ with libasan and the ROCm runtime are needed")
    lib = build.build_host_sanitized()
    env = dict(os.environ)
    env.update(H3DIT_LIB=lib, LD_PRELOAD=asan,
               # the Python interpreter and the ROCm runtime are not instrumented:
               # their allocations are not ours to account for
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
