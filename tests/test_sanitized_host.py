"""The host layer of the C ABI and the oracle under AddressSanitizer + UndefinedBehaviorSanitizer.

Builds libmoe_san.so (host code instrumented, device code as usual) and liboracle_san.so, then
runs the ABI validation tests and the oracle's pins in a child process that preloads clang's
sanitizer runtime and loads the instrumented libraries in place of the usual ones. Any report
(heap overflow, use after free, signed overflow, misaligned or out-of-bounds access, invalid
shift) aborts the child, which fails this test. CPU only: no call reaches a kernel.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_layer_and_oracle_under_sanitizers():
    from mixture_experts_ffn_softmax_amd import build as hip_build
    import oracle

    runtime = hip_build.sanitizer_runtime()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("clang's ASan runtime is not installed")
    lib = hip_build.build(sanitize=True)
    olib = oracle.build_sanitized()
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime + ((" " + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:alloc_dealloc_mismatch=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["MOE_LIBRARY"] = lib
    env["MOE_ORACLE_LIBRARY"] = olib
    tests = ["tests/test_abi.py", "tests/test_oracle_route.py", "tests/test_oracle_permute.py",
             "tests/test_oracle_fp8.py", "tests/test_oracle_fp4.py",
             "tests/test_oracle_precision.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", *tests], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
