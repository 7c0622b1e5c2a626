"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host side of
the library (hipcc, sanitizers on the host pass only) and of the oracle
(clang), exercised on the CPU by tests/sanitizer_driver.py in a child
process with the shared ASan runtime preloaded.  Any report fails the test
(UBSan does not recover).  The device code is not instrumented."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and _asan_runtime()),
                    reason="ROCm clang with the ASan runtime is not installed")
def test_host_library_and_oracle_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libe2ttt_san.so")
    orc = str(tmp_path / "liboracle_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libasan"]
    csrc = os.path.join(ROOT, "chunk_weight_update_amd", "csrc")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops"] + san +
                   ["-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", lib,
                    os.path.join(csrc, "e2ttt.hip")], check=True, capture_output=True)
    subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-shared-libasan", "-ffp-contract=off",
                    "-shared", "-fPIC", "-std=c99", "-o", orc,
                    os.path.join(ROOT, "oracle", "e2ttt_oracle.c"), "-lm"],
                   check=True, capture_output=True)
    driver = os.path.join(ROOT, "tests", "sanitizer_driver.py")
    ref = str(tmp_path / "ref.npz")
    env = dict(os.environ, PYTHONPATH=ROOT)
    subprocess.run([sys.executable, driver, ref, "write"], env=env, check=True,
                   capture_output=True)
    env.update(E2TTT_LIBRARY=lib, E2TTT_ORACLE_LIBRARY=orc, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([sys.executable, driver, ref], env=env, capture_output=True, text=True)
    report = res.stdout + res.stderr
    assert res.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert "sanitizer driver: ok" in report
