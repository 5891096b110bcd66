"""The C ABI's host code under AddressSanitizer.

libmla_hostcheck.so is libmla.so built with -fsanitize=address on its host code (the
device code is the same).  Every test of tests/test_abi.py (exports, status strings,
workspace sizing, the host-side rejections of every entry point) runs against it in a
child process that preloads the compiler's ASan runtime, so an out-of-bounds access or
a use after free in argument checking, sizing or the status table fails this test.
No GPU is used: nothing the host checks accept is ever enqueued.
"""
import os
import subprocess
import sys

import pytest

from mla_latent_kv_16_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Runs tests/test_abi.py with the binding pointed at the sanitized library; LD_PRELOAD
# is dropped from the environment of any process the tests start (nm, the C compiler).
_DRIVER = r"""
import os, sys
os.environ.pop("LD_PRELOAD", None)
sys.path.insert(0, {root!r})
import mla_latent_kv_16_amd as mla
from mla_latent_kv_16_amd import _binding
_binding.LIB_PATH = mla.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {test!r}]))
"""


def test_host_checks_under_address_sanitizer():
    if not os.path.exists(build.HOSTCHECK_LIB):
        pytest.fail(f"{build.HOSTCHECK_LIB} is missing: build it with "
                    "`python -m mla_latent_kv_16_amd.build`")
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.asan_runtime()
    # Python itself is not instrumented and keeps memory until exit: leaks are not errors
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    code = _DRIVER.format(root=ROOT, lib=build.HOSTCHECK_LIB,
                          test=os.path.join(ROOT, "tests", "test_abi.py"))
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=600, cwd=ROOT)
    out = res.stdout + res.stderr
    print(out[-4000:])
    assert "AddressSanitizer" not in out, "AddressSanitizer reported an error"
    assert res.returncode == 0, f"test_abi.py under ASan exited with {res.returncode}"
    assert " passed" in out
