"""The C-ABI host tests again, against a build whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only). The argument checks,
planners and workspace-size arithmetic run in the sanitized library; any invalid
memory access or undefined operation aborts the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def test_abi_host_tests_pass_under_host_sanitizers():
    from learned_chunk_routed_amd import build as B
    lib = B.build_sanitized()
    runtime = B.sanitizer_runtime()
    syms = subprocess.run(["nm", "-D", lib], stdout=subprocess.PIPE, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    runner = (
        "import sys\n"
        "import learned_chunk_routed_amd._lib as L\n"
        f"L.LIB_PATH = {lib!r}\n"
        "L.load()\n"
        "maps = open('/proc/self/maps').read()\n"
        "assert 'libclang_rt.asan' in maps and 'liblcr_sanitized.so' in maps\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi_host.py']))\n")
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", runner], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
