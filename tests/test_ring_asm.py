"""The streaming expert kernel keeps its weight loads in flight in registers
(inline-assembly loads, explicit vmcnt waits).  The compiler believes such a
register is written when the load issues, so a copy or reuse of it before the
wait reads stale data.  These tests compile the kernel for gfx950 and check its
assembly on every control-flow path (tests/asm_ring_check.py)."""
import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "w4a16_routed_expert_router_amd"))

import asm_ring_check as arc  # noqa: E402

# A ring of two register slots around a loop (each wait retires the older
# slot), once with a copy of the younger, still in-flight slot on the back
# edge (the pattern a failed register coalescing produces) and once without.
_GOOD = """
_Zgood:                                 ; @_Zgood
	;;#ASMSTART
	global_load_dwordx4 v[8:11], v[20:21], off
	;;#ASMEND
.LBB0_1:
	;;#ASMSTART
	global_load_dwordx4 v[4:7], v[20:21], off
	;;#ASMEND
	;;#ASMSTART
	s_waitcnt vmcnt(1)
	;;#ASMEND
	v_add_u32_e32 v14, v8, v9
	;;#ASMSTART
	global_load_dwordx4 v[8:11], v[20:21], off
	;;#ASMEND
	;;#ASMSTART
	s_waitcnt vmcnt(1)
	;;#ASMEND
	v_add_u32_e32 v15, v4, v5
	s_cbranch_scc1 .LBB0_1
	s_endpgm
.Lfunc_end0:
"""
_BAD = _GOOD.replace("_Zgood", "_Zbad").replace(
    "\tv_add_u32_e32 v15, v4, v5\n", "\tv_add_u32_e32 v15, v4, v5\n\tv_mov_b64_e32 v[12:13], v[8:9]\n")


def test_checker_flags_a_copy_of_an_inflight_register():
    bad = arc.kernel_bodies(_BAD)["_Zbad"]
    hz = arc.check(bad)
    assert [h[1] for h in hz] == ["v_mov_b64_e32 v[12:13], v[8:9]"], hz
    good = arc.kernel_bodies(_GOOD)["_Zgood"]
    assert arc.check(good) == []


def test_checker_retires_only_loads_older_than_the_wait_count():
    # vmcnt(1) leaves the youngest load in flight: a read of its register is a hazard
    asm = """
_Zw:                                    ; @_Zw
	;;#ASMSTART
	global_load_dwordx4 v[0:3], v[20:21], off
	;;#ASMEND
	;;#ASMSTART
	global_load_dwordx4 v[4:7], v[20:21], off
	;;#ASMEND
	s_waitcnt vmcnt(1)
	v_add_u32_e32 v10, v0, v1
	v_add_u32_e32 v11, v4, v1
	s_endpgm
.Lfunc_end0:
"""
    hz = arc.check(arc.kernel_bodies(asm)["_Zw"])
    assert [h[1] for h in hz] == ["v_add_u32_e32 v11, v4, v1"], hz


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
def test_stream_kernel_ring_registers_untouched_until_waited(tmp_path):
    import build_lib as bl
    src = os.path.join(bl.CSRC, "expert_stream.hip")
    flags = [f for f in bl.HIP_FLAGS if f != "-fPIC"] + ["-I", bl.CSRC]
    asm = arc.compile_asm(bl.hipcc(), flags, src, str(tmp_path / "stream.s"))
    bodies = {k: v for k, v in arc.kernel_bodies(asm).items() if "stream_expert_kernel" in k}
    assert len(bodies) == 3, sorted(bodies)
    for name, body in bodies.items():
        assert arc.check(body) == [], name
