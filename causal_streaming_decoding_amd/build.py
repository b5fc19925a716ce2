"""Build libwedlm.so (gfx950) from the HIP sources with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in parallel)
and the objects are linked into ``libwedlm.so`` next to this file. The build
always recompiles. Packed fp32 VALU instructions are switched off for the
device code (``-packed-fp32-ops``); the host pass warns that it does not know
that feature, which is harmless. The compiler's intermediate files, the device
assembly among them, stay in ``_build/``: before linking, ``isa_audit`` checks
there that no register loaded by an inline-asm load is read, copied or reused
before the counted wait that retires the load, and the build fails if one is.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

try:
    from . import isa_audit
except ImportError:  # run as a script
    import isa_audit

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libwedlm.so")
ARCH = os.environ.get("WEDLM_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-file additions. attn.hip, block_attn.hip: no NaN reaches a maximum or
# comparison there (scores of invisible keys are set to -inf before any
# maximum), so the compiler need not quiet NaN operands before every v_max_f32;
# entropy_chunks.hip (and the chunk blocks in attn.hip's launch): the logits are
# taken to be finite. Files with host-side NaN checks of arguments keep the
# default.
FILE_CFLAGS = {"attn.hip": ["-fno-honor-nans"], "block_attn.hip": ["-fno-honor-nans"],
               "entropy_chunks.hip": ["-fno-honor-nans"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_CFLAGS.get(os.path.basename(src), []), "-save-temps=obj", "-c",
           src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(verbose=False, jobs=8):
    """Compile every HIP source and link libwedlm.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources()))
    found = isa_audit.audit_dir(BUILD_DIR)
    if found:
        lines = "\n".join(f"  {fn} line {ln}: {text} touches {regs}" for fn, ln, text, regs in found[:20])
        raise RuntimeError("device code reads registers of inline-asm loads still in flight:\n" + lines)
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
