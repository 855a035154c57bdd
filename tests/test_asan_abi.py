"""The C ABI's host code under AddressSanitizer (CPU).

Builds the library with its host code (argument validation, workspace
layout, launch sequence, error reporting) compiled with -fsanitize=address,
then runs tests/test_abi.py against that build in a child process with the
ASan runtime preloaded.  Any invalid host memory access (out-of-bounds read
of a struct, use after free of the error string, ...) aborts the child with
an ASan report, which fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_clean_under_asan():
    from hybrid_attention_ssm_amd.csrc import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    lib = B.build_asan(jobs=min(8, os.cpu_count() or 1))
    rt = B.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env.update(HH_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0")
    env.pop("HH_FAULT_INJECT", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
    assert " passed" in out
