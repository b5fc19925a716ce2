"""The device-assembly audit of inline-asm loads (CPU).

The audit replays a function in program order with a queue of vector-memory
operations that s_waitcnt vmcnt(N) retires from the front; an instruction that
names a destination register of an inline-asm load still in the queue is a
finding. These cases pin that replay on small hand-written listings, then run
it over the device assembly of the current build (when the build has left it).
"""

import os

import pytest

from causal_streaming_decoding_amd import isa_audit
from causal_streaming_decoding_amd.build import BUILD_DIR


def _fn(body):
    return body.strip("\n").splitlines()


ASM_LOAD = """
  ;;#ASMSTART
  global_load_dwordx4 v[10:13], v[2:3], off nt
  ;;#ASMEND
"""


def test_use_after_the_counted_wait_is_clean():
    lines = _fn(ASM_LOAD + """
  ;;#ASMSTART
  s_waitcnt vmcnt(0) lgkmcnt(0)
  ;;#ASMEND
  v_mfma_f32_32x32x16_bf16 a[0:15], v[10:13], v[20:23], a[0:15]
""")
    assert isa_audit.audit_function(lines) == []


def test_copy_before_the_wait_is_found():
    lines = _fn(ASM_LOAD + """
  v_mov_b64_e32 v[40:41], v[12:13]
  s_waitcnt vmcnt(0)
""")
    found = isa_audit.audit_function(lines)
    assert len(found) == 1 and found[0][3] == [("v", 12), ("v", 13)]


def test_reuse_as_an_address_before_the_wait_is_found():
    lines = _fn(ASM_LOAD + """
  v_add_u32_e32 v11, 64, v5
  global_load_dword v7, v[10:11], off
""")
    assert len(isa_audit.audit_function(lines)) == 2  # the write of v11, then its use as an address


def test_waits_retire_in_issue_order():
    # two asm loads, then a compiler load: vmcnt(2) retires only the first
    lines = _fn(ASM_LOAD + """
  ;;#ASMSTART
  global_load_dwordx4 v[14:17], v[4:5], off nt
  ;;#ASMEND
  global_load_dword v30, v[6:7], off
  s_waitcnt vmcnt(2)
  v_mov_b32_e32 v40, v10
  v_mov_b32_e32 v41, v14
  s_waitcnt vmcnt(0x1)
  v_mov_b32_e32 v42, v15
""")
    found = isa_audit.audit_function(lines)
    assert [f[2] for f in found] == ["v_mov_b32_e32 v41, v14"]


def test_compiler_loads_and_dma_are_not_checked():
    # the compiler places its own waits; a DMA into LDS writes no register
    lines = _fn("""
  global_load_dwordx4 v[10:13], v[2:3], off
  global_load_lds_dwordx4 v[4:5], off
  v_mov_b32_e32 v40, v10
  s_waitcnt 0
""")
    assert isa_audit.audit_function(lines) == []


def test_a_later_load_into_the_same_registers_is_allowed():
    lines = _fn(ASM_LOAD + """
  ;;#ASMSTART
  global_load_dwordx4 v[10:13], v[6:7], off nt
  ;;#ASMEND
  s_waitcnt vmcnt(0)
  v_mov_b32_e32 v40, v10
""")
    assert isa_audit.audit_function(lines) == []


def test_audit_file_splits_functions(tmp_path):
    p = tmp_path / "k-hip-amdgcn-amd-amdhsa-gfx950.s"
    p.write_text("\n".join([
        "_Z1av:", ";;#ASMSTART", "  global_load_dword v1, v[2:3], off", ";;#ASMEND",
        "  v_mov_b32_e32 v4, v1", ".Lfunc_end0:",
        "_Z1bv:", "  v_mov_b32_e32 v4, v1", ".Lfunc_end1:", ""]))
    found = isa_audit.audit_file(str(p))
    assert [(f[0].split(":")[1], f[1]) for f in found] == [("_Z1av", 5)]


def test_current_build_is_clean():
    files = isa_audit.device_assembly(BUILD_DIR)
    if not files:
        pytest.skip("no device assembly in the build folder (build the library first)")
    assert any(os.path.basename(f).startswith("lm_head") for f in files)
    assert isa_audit.audit_dir(BUILD_DIR) == []
