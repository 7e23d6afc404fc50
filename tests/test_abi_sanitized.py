"""The C-ABI contract checks (tests/test_abi.py) against a build of the library
whose host code (dg_api.cpp: argument checking, workspace layout, status
strings) runs under AddressSanitizer and UndefinedBehaviorSanitizer. CPU only:
every call checked there returns before any HIP call. Any sanitizer report
aborts the child process and fails this test."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    path = os.path.join(ROOT, "discrete_diffusion_decoding_dg_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_dg_build_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.slow
def test_abi_contract_under_asan_and_ubsan(tmp_path):
    b = _build_module()
    runtime = b.sanitizer_runtime()
    if not os.path.exists(runtime):
        pytest.skip(f"no ASan runtime at {runtime!r}")
    lib = b.build_sanitized(str(tmp_path))
    env = dict(os.environ, LD_PRELOAD=runtime, DG_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout
