"""The C ABI's host code under AddressSanitizer (no GPU needed).

Builds every translation unit of the library with AddressSanitizer on its host
code only (the device code is compiled as usual), links the test program
tests/abi_asan_driver.cpp against it and runs it: each of its calls is refused
by host-side validation before any HIP call, so the run checks that argument
validation and error reporting of every entry point stay inside their memory."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "learned_token_pruning_03_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
SOURCES = ["tg_api.cpp", "gate.hip", "select.hip", "gather.hip", "rope.hip", "attn.hip", "decode.hip", "dense.hip"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_abi_validation_is_clean_under_address_sanitizer():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    # Sanitizer flags apply to the host compilation only.
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    hip_flags = ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

    def compile_one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *hip_flags, *common, *san, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, f"{src}:\n{res.stderr[-2000:]}"
        return obj

    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    drv_obj = os.path.join(OUT, "driver.o")
    res = subprocess.run([hipcc, *common, *san, "-c", os.path.join(ROOT, "tests", "abi_asan_driver.cpp"), "-o",
                          drv_obj], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    exe = os.path.join(OUT, "abi_asan_driver")
    res = subprocess.run([hipcc, "--offload-arch=gfx950", *san, drv_obj, *objs, "-o", exe], capture_output=True,
                         text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert "0 mismatches" in run.stdout
