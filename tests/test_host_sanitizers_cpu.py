"""The library's host code under the address and undefined-behaviour sanitizers (CPU).

Every HIP source is compiled with the sanitizers on its host side only (the
device code is built as usual and never runs here), linked into a separate
library in a temporary folder, and driven by `tests/host_asan/abi_sanitized.c`:
status strings, the size queries swept over extreme shapes (one argument at a
time from INT_MIN to INT_MAX) and, for every entry point, calls that must fail
their argument checks before anything is launched. The run fails on any
sanitizer report (a signed overflow in the plan arithmetic, an out-of-bounds
host access) or any unexpected status.
"""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from causal_streaming_decoding_amd import build as B

pytestmark = pytest.mark.slow

CLANG = "/opt/rocm/llvm/bin/clang"
DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host_asan", "abi_sanitized.c")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(B.HIPCC) and os.path.exists(CLANG)),
                    reason="hipcc / clang not available")
def test_host_code_under_sanitizers(tmp_path):
    flags = [f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{B.INCLUDE}", f"-I{B.CSRC}"]

    def cc(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        extra = B.FILE_CFLAGS.get(os.path.basename(src), [])
        r = subprocess.run([B.HIPCC, *flags, *extra, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(cc, B.sources()))
    lib = str(tmp_path / "libwedlm_san.so")
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_SAN[:4],
                        *objs, "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_sanitized")
    r = subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-omit-frame-pointer", f"-I{B.INCLUDE}", DRIVER,
                        f"-L{tmp_path}", "-lwedlm_san", f"-Wl,-rpath,{tmp_path}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0"  # the HIP runtime keeps its allocations to exit
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout + r.stderr)[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
