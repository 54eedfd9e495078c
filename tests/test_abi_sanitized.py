"""librr's host code (argument checks, workspace sizes, status strings)
under AddressSanitizer and UndefinedBehaviorSanitizer: rr_api.hip is rebuilt
with the sanitizers on its host side only, linked with the library's other
objects, and driven by tests/sanitize/abi_driver.c (CPU only; nothing is
enqueued on a GPU)."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_prefill_rr_amd", "csrc")
BUILD = os.path.join(ROOT, "long_context_prefill_rr_amd", "_build")


@pytest.mark.skipif(shutil.which("hipcc") is None or shutil.which("gcc") is None,
                    reason="hipcc and gcc needed")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    objs = [o for o in glob.glob(os.path.join(BUILD, "*.o")) if not o.endswith("rr_api.o")]
    if len(objs) < 6:
        from long_context_prefill_rr_amd import build
        build.build()
        objs = [o for o in glob.glob(os.path.join(BUILD, "*.o")) if not o.endswith("rr_api.o")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api = str(tmp_path / "api.o")
    subprocess.run(["hipcc", "-c", os.path.join(CSRC, "rr_api.hip"), "-o", api, "-O1", "-g",
                    "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
                   + san, check=True, capture_output=True, text=True)
    drv = str(tmp_path / "drv.o")
    subprocess.run(["gcc", "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), "-o", drv,
                    "-g", "-I", os.path.join(ROOT, "include"), "-fsanitize=address,undefined"],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "abi_driver")
    subprocess.run(["hipcc", "-o", exe, drv, api] + objs + ["--offload-arch=gfx950"] + san,
                   check=True, capture_output=True, text=True)
    # Leak checking is off: the HIP runtime keeps its own allocations to exit.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"
