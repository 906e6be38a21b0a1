"""The C ABI's argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer: the host code of libtokengate.so built with both
(build.py --sanitize; device code as usual), and the whole ABI test module run
against that build in a child process with the ASan runtime preloaded. Any
out-of-bounds access, use after free or undefined behaviour in the host code
those tests reach ends the child with a report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from learned_token_pruning_post_amd import build  # noqa: E402


def test_abi_validation_under_asan_and_ubsan():
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    lib = build.build(verbose=False, sanitize=True)
    rt = build.asan_runtime()
    # the library really is instrumented (it calls into the ASan runtime)
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True)
    assert "__asan_report" in nm.stdout and "__ubsan_handle" in nm.stdout
    env = dict(os.environ, TG_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout and "failed" not in r.stdout, out
