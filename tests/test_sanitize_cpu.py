"""The host side of the library (argument validation, workspace sizing, the
persistent-image arithmetic) under AddressSanitizer and
UndefinedBehaviorSanitizer: the sanitizer build of the host code
(build.py --sanitize) runs the C-ABI validation tests of test_abi_cpu.py in a
child process with the ASan runtime preloaded; any report fails the test.
No GPU is used (every call there is rejected or only sizes things)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(_asan_runtime() is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc and the clang ASan runtime")
def test_host_validation_under_asan_and_ubsan():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_csa2_build", os.path.join(ROOT, "sparse_attention_fp4_e2m1_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    lib = mod.build(verbose=False, sanitize=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "CSA2_LIBRARY": lib,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "passed" in out
    # the child really loaded the sanitizer build
    probe = subprocess.run([sys.executable, "-c",
                            "import sparse_attention_fp4_e2m1_amd.csa2 as b; print(b.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip().endswith("libcsa2_sanitize.so"), probe.stdout + probe.stderr
