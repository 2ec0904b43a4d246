"""The C ABI's host code under AddressSanitizer (CPU): the library built with its host side
instrumented (`python -m sparse_moe_transformer_router_amd.build --asan`; the GPU code is built as
always), loaded into a process that preloads the sanitizer runtime, runs the ABI's CPU tests
(argument checks and error paths of every entry point, workspace sizes, exported symbols). Any
sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_under_host_asan():
    from sparse_moe_transformer_router_amd import build as b
    lib = b.build(asan=True)
    rt = b.asan_runtime()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("the compiler's shared AddressSanitizer runtime is not installed")
    preload = ":".join(p for p in (rt, os.environ.get("LD_PRELOAD", "")) if p)  # the runtime must come first
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0", MOE_MXFP4_LIBRARY=lib)
    check = "import sparse_moe_transformer_router_amd._lib as L; L.lib(); print(L.LIB_PATH)"
    r = subprocess.run([sys.executable, "-c", check], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().splitlines()[-1] == lib, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
