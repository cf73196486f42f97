"""The C ABI's host code under AddressSanitizer: the CPU tests of the ABI
(tests/test_abi.py: exports, argument validation, status codes, the debug
switch) run again in a child process against a build of the same sources
with AddressSanitizer on the host code, its runtime preloaded.  Any invalid
host memory access in the validation or workspace paths fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_address_sanitizer():
    sys.path.insert(0, ROOT)
    from mla_latent_kv_07_amd import build as b
    try:
        rt = b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = b.build_asan()
    env = dict(os.environ)
    env.update(MLA_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
