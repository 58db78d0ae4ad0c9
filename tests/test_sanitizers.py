"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two builds of the same sources: the library with both sanitizers on its host
code (argument validation and launchers; `top_indexer_sparse_amd/build.py
--sanitize`, device code unchanged) and the oracle (`oracle/build.py
--sanitize`).  The ABI tests run against the first with clang's ASan runtime
preloaded, the oracle's pins against the second with gcc's runtimes; any
report aborts the run (no recovery), so a clean exit is the check.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env_extra, test_file):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", test_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_library_host_code_under_asan_ubsan():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang ASan runtime not found")
    sys.path.insert(0, ROOT)
    from top_indexer_sparse_amd import build
    lib = build.build(sanitize=True)
    out = _run({"LD_PRELOAD": rt[-1], "SA_LIB": lib}, "test_abi.py")
    assert " passed" in out


def test_oracle_under_asan_ubsan():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                           text=True).stdout.strip()
    if not (os.path.isabs(asan) and os.path.isabs(ubsan)):
        pytest.skip("gcc sanitizer runtimes not found")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(sanitize=True)
    out = _run({"LD_PRELOAD": f"{asan} {ubsan}", "SA_ORACLE_LIB": lib}, "test_oracle_pins.py")
    assert " passed" in out
