"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer: libmsa is rebuilt with its host code instrumented
(device code unchanged; nothing is launched), and test_abi_cpu.py runs in a
child process against that build with the ASan runtime preloaded."""

import glob
import os
import subprocess
import sys

import pytest

from sparse_retrieval_memory_amd import build

ASAN_RT = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not ASAN_RT or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc or the clang ASan runtime is not installed")
def test_abi_validation_under_host_sanitizers(tmp_path):
    lib = build.build_sanitized(str(tmp_path / "libmsa_sanitized.so"))
    env = dict(os.environ)
    # the sanitizer runtime must come first; anything already preloaded stays
    env["LD_PRELOAD"] = ":".join([ASAN_RT[-1]] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["MSA_LIBRARY"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(REPO, "tests", "test_abi_cpu.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], env=env, cwd=REPO, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
