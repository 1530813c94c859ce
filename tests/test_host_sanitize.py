"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libcsa2 is compiled for gfx950 with the sanitizers on the
host compilation pass only (`-Xarch_host`), and linked with
`tests/host_abi_driver.c`, which drives the validation
of every entry point, the workspace-size arithmetic and the trace calls.  The
driver makes calls that pass validation only when the HIP runtime reports no
device (their pointers are host memory; the launches then fail with a HIP
error); the test hides every GPU from it.
"""

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp4_kv_cache_index_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _host_flags():
    out = []
    for f in SAN:
        out += ["-Xarch_host", f]
    return out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not present")
def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    tmp = tempfile.mkdtemp(prefix="csa2_san_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-Wno-unused-command-line-argument"] + _host_flags() + \
                  ["-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj

        with ThreadPoolExecutor(4) as ex:
            objs = list(ex.map(compile_one, ["quant.hip", "select.hip", "score.hip", "attn.hip", "api.cpp"]))
        drv = os.path.join(tmp, "driver.o")
        r = subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-I", os.path.join(ROOT, "include")] + SAN +
                           ["-c", os.path.join(ROOT, "tests", "host_abi_driver.c"), "-o", drv],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        exe = os.path.join(tmp, "host_abi_driver")
        r = subprocess.run([CLANGXX] + SAN + [drv] + objs +
                           ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ)
        env.update({
            "HIP_VISIBLE_DEVICES": "-1", "ROCR_VISIBLE_DEVICES": "-1", "CUDA_VISIBLE_DEVICES": "-1",
            # the HIP runtime's own allocations at exit are not this library's
            "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        })
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        log = r.stdout + r.stderr
        assert r.returncode == 0, log[-4000:]
        assert "runtime error" not in log and "AddressSanitizer" not in log, log[-4000:]
        assert "0 failed" in r.stdout, log[-4000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
