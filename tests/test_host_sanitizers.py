"""The host C++ of the library -- block manager, scheduler, step packer and
work planner, which do raw index arithmetic into caller buffers -- built with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code only), and the
host parity tests re-run against that build in a child process: every
out-of-bounds access, use after free or undefined operation they reach aborts
the run.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_346_amd", "csrc")
HOST_SOURCES = ["block_manager.cpp", "scheduler.cpp", "step_pack.cpp", "plan.cpp", "status.cpp"]
PARITY_TESTS = ["tests/test_block_manager_parity.py", "tests/test_scheduler_parity.py",
                "tests/test_step_pack.py", "tests/test_plan.py"]


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if _runtime("libasan.so") is None or _runtime("libubsan.so") is None:
        pytest.skip("g++ sanitizer runtimes not installed")
    out = str(tmp_path_factory.mktemp("san") / "libpkv_host_san.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           *[os.path.join(CSRC, s) for s in HOST_SOURCES], "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_host_parity_under_sanitizers(sanitized_lib):
    env = dict(os.environ)
    env.update(PKV_TEST_HOST_LIB=sanitized_lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PARITY_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
