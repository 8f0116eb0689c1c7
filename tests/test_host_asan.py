"""The C ABI's host code (argument validation, workspace planning, dispatch up
to the first launch) under AddressSanitizer, on the CPU.

The library is built host-only with ASan instrumentation (no device code: the
validation paths return before any launch), the compiler's sanitizer runtime is
preloaded, and the ABI tests of tests/test_abi.py run against that build in a
child process. Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

from sparse_attention_indexer_block_amd.build import asan_runtime, build_host_asan

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

RUNNER = r"""
import sys
import sparse_attention_indexer_block_amd as S
S.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-m", "not gpu", "-p", "no:cacheprovider", sys.argv[2]]))
"""


@pytest.mark.slow
def test_abi_validation_under_host_asan(tmp_path):
    rt = asan_runtime()
    if not rt:
        pytest.skip("the toolchain has no AddressSanitizer runtime")
    lib = build_host_asan(str(tmp_path))
    env = dict(os.environ)
    # the sanitizer runtime must come first; anything already preloaded stays
    env["LD_PRELOAD"] = rt + (os.pathsep + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:exitcode=86"
    env["PYTHONPATH"] = os.pathsep.join(p for p in (ROOT, HERE, env.get("PYTHONPATH", "")) if p)
    r = subprocess.run([sys.executable, "-c", RUNNER, lib, os.path.join(HERE, "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-4000:]
