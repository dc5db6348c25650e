"""The C ABI's host-side argument checks under AddressSanitizer (CPU only).

The library is rebuilt with the host pass instrumented (device code unchanged) into
_build/libfa_asan_host.so, and tests/test_contract.py runs against it in a child process with
the ASan runtime preloaded: every entry point's rejection paths, the workspace-size and
split-count helpers and fa_strerror execute under ASan, which aborts the child on any
out-of-bounds or use-after-free access."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from exact_attention_06_amd import build as B  # noqa: E402

SOURCES = [os.path.join(ROOT, "exact_attention_06_amd", "csrc", n)
           for n in os.listdir(os.path.join(ROOT, "exact_attention_06_amd", "csrc"))] + \
          [os.path.join(ROOT, "include", "fa_fwd.h")]


def _stale():
    if not os.path.exists(B.ASAN_LIB):
        return True
    t = os.path.getmtime(B.ASAN_LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES)


@pytest.mark.slow
def test_contract_suite_under_host_asan():
    if not os.path.exists(B.hipcc()):
        pytest.skip("hipcc not found")
    if _stale():
        B.build_asan_host()
    env = dict(os.environ, LD_PRELOAD=B.asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               FA_LIB=B.ASAN_LIB)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_contract.py")], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    print(tail)
    assert res.returncode == 0 and "AddressSanitizer" not in tail, tail
