"""The oracle and the library's host-side code under AddressSanitizer and
UndefinedBehaviorSanitizer. Each is rebuilt with the sanitizers and the CPU
tests that drive it run again in a child process that preloads the matching
runtime: gcc's libasan for the oracle (built with gcc), clang's for the HIP
library's host code (built with hipcc; device code is not instrumented and
not run). Any report aborts the child, failing the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env_extra, tests, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", t) for t in tests]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build(force=True, sanitize=True, out=str(tmp_path / "libtt_oracle_san.so"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's libasan is not installed")
    out = _run({"LD_PRELOAD": asan, "TT_ORACLE_LIB": lib},
               ["test_oracle_forward.py", "test_oracle_backward.py"], timeout=600)
    assert "passed" in out


def test_library_host_code_under_asan_ubsan(tmp_path):
    from tensor_train_compressed_amd import build as b
    lib = b.build_host_sanitized(str(tmp_path))
    out = _run({"LD_PRELOAD": b.asan_runtime(), "TT_EMB_LIBRARY": lib},
               ["test_abi_host.py"], timeout=300)
    assert "passed" in out
