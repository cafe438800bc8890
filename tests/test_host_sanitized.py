"""The host-side library checks (tests/test_lib_host.py: descriptor checks, arena layout of every
model variant, refusals, cut arithmetic) run again against a build whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer; any sanitizer report fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "_build", "libbvf_san.so")
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.mark.skipif(not os.path.exists(SAN_LIB), reason="host-sanitized library not built (__graft_entry__.build())")
@pytest.mark.skipif(not RUNTIME, reason="no AddressSanitizer runtime in /opt/rocm/llvm")
def test_host_code_under_address_and_ub_sanitizers():
    code = ("import sys\n"
            "from block_verify_forward_amd import bvf\n"
            f"bvf.LIB_PATH = {SAN_LIB!r}\n"
            "import pytest\n"
            "sys.exit(pytest.main(['tests/test_lib_host.py', '-q', '-p', 'no:cacheprovider']))\n")
    env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
