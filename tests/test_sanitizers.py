"""Host-side sanitizer runs (CPU only; opt-in, DSA_IDX_SANITIZE=1, since the library build takes a
minute or two):

* oracle.c built with gcc's AddressSanitizer + UndefinedBehaviorSanitizer, and every oracle pin
  test run against it;
* libdsaidx built with host-only ASan + UBSan (device code unchanged), and the C-ABI tests run
  against it: argument validation, workspace sizing, the architecture check and the symbol
  table, all on the host.

Each run is a child process with the sanitizer runtime preloaded; it must pass and print no
sanitizer report.  Leak checking is off: the Python interpreter itself is not instrumented.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(os.environ.get("DSA_IDX_SANITIZE") != "1",
                                reason="sanitizer builds are opt-in: set DSA_IDX_SANITIZE=1")
REPORT = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run(env_extra, tests):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("DSA_IDX_SANITIZE", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1800)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in REPORT:
        assert marker not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan():
    import oracle
    so = oracle.build_sanitized()
    gcc = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ub = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    out = _run({"ORACLE_LIB": so, "LD_PRELOAD": f"{gcc} {ub}"}, tests)
    print(out.splitlines()[-1])


def test_c_abi_under_asan_ubsan():
    from sparse_attention_token_idx_amd import build as B
    so = B.build(sanitize=True)
    out = _run({"DSA_IDX_LIB": so, "LD_PRELOAD": B.sanitizer_runtime()},
               [os.path.join(ROOT, "tests", "test_abi.py")])
    print(out.splitlines()[-1])
