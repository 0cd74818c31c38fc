"""The C ABI's host code (argument checks, workspace layout, launch set-up)
under AddressSanitizer and UndefinedBehaviorSanitizer: build.py builds a copy
of the library with the sanitizers on its host code, and the ABI checks of
test_abi.py run against it in a child process with the sanitizer runtime
preloaded.  Any sanitizer report ends that process with an error.  CPU only:
these checks never launch a kernel."""
import os
import pathlib
import shutil
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
SAN_LIB = ROOT / "packed_varlen_attention_amd" / "_build_san" / "libmf.so"


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_abi_checks_pass_under_host_sanitizers():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    r = subprocess.run([sys.executable, "-m", "packed_varlen_attention_amd.build", "--sanitize-host"], cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-3000:]
    assert SAN_LIB.exists()
    runtime = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True).stdout.strip()
    if not runtime or not os.path.exists(runtime):
        pytest.skip("sanitizer runtime not found")
    env = dict(os.environ, MF_LIBRARY=str(SAN_LIB), LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", str(ROOT / "tests" / "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
