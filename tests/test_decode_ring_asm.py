"""The decode kernel's inline-asm load ring, checked on the built assembly.

The E4M3 decode keeps its K/V loads in flight in registers the compiler does
not know are being written by memory (inline global_load_dwordx4, explicit
vmcnt waits).  fp8_e4m3_scaled_amd/ring_check.py (also run by every library
build) proves from the assembly that no instruction
reads, copies or reuses such a register before its wait; these tests first
show that the checker catches each kind of mistake on small hand-written
listings, then run it over every E4M3 decode instance of the library source,
compiled with the library's own flags.
"""
from __future__ import annotations

import importlib.util
import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load(name, rel):
    spec = importlib.util.spec_from_file_location(name, os.path.join(ROOT, rel))
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod                  # dataclasses look their module up by name
    spec.loader.exec_module(mod)
    return mod


ring_asm = _load("kvfp8_ring_check", os.path.join("fp8_e4m3_scaled_amd", "ring_check.py"))


def _listing(body: str) -> list[str]:
    return body.strip("\n").splitlines()


GOOD = """
    v_mov_b32 v10, 0
    ;;#ASMSTART
    global_load_dwordx4 v[0:3], v[10:11], off
    ;;#ASMEND
    ;;#ASMSTART
    global_load_dwordx4 v[4:7], v[10:11], off
    ;;#ASMEND
    ;;#ASMSTART
    s_waitcnt vmcnt(1)
    ;;#ASMEND
    v_add_f32 v20, v0, v1
    ;;#ASMSTART
    s_waitcnt vmcnt(0)
    ;;#ASMEND
    v_add_f32 v21, v4, v5
    s_endpgm
"""


def test_checker_accepts_a_sound_ring():
    v, n = ring_asm.check(_listing(GOOD))
    assert n == 2 and v == []


def test_checker_flags_a_copy_before_the_wait():
    bad = GOOD.replace("    ;;#ASMSTART\n    s_waitcnt vmcnt(1)", "    v_mov_b32 v30, v2\n    ;;#ASMSTART\n    s_waitcnt vmcnt(1)")
    v, _ = ring_asm.check(_listing(bad))
    assert len(v) == 1 and "v_mov_b32 v30, v2" in v[0]


def test_checker_flags_a_reuse_while_in_flight():
    bad = GOOD.replace("v_add_f32 v20, v0, v1", "v_add_f32 v20, v0, v1\n    v_mov_b32 v6, 0")
    v, _ = ring_asm.check(_listing(bad))
    assert len(v) == 1 and "v_mov_b32 v6, 0" in v[0]


def test_checker_counts_waits_in_issue_order():
    # vmcnt(1) retires only the older load: the younger one is still pending
    bad = GOOD.replace("v_add_f32 v20, v0, v1", "v_add_f32 v20, v0, v4")
    v, _ = ring_asm.check(_listing(bad))
    assert len(v) == 1 and "[4]" in v[0]


def test_checker_follows_a_branch_that_skips_the_wait():
    bad = """
    ;;#ASMSTART
    global_load_dwordx4 v[0:3], v[10:11], off
    ;;#ASMEND
    s_cbranch_scc1 .LBB0_2
    ;;#ASMSTART
    s_waitcnt vmcnt(0)
    ;;#ASMEND
.LBB0_2:
    v_add_f32 v20, v0, v1
    s_endpgm
"""
    v, _ = ring_asm.check(_listing(bad))
    assert len(v) == 1 and "v_add_f32 v20, v0, v1" in v[0]


def test_checker_follows_a_loop_back_edge():
    # the load issued at the bottom of the body is still in flight when the
    # next iteration's top reuses its register
    bad = """
    s_mov_b32 s0, 4
.LBB0_1:
    v_mov_b32 v2, 0
    ;;#ASMSTART
    global_load_dwordx4 v[0:3], v[10:11], off
    ;;#ASMEND
    s_sub_u32 s0, s0, 1
    s_cbranch_scc1 .LBB0_1
    s_waitcnt vmcnt(0)
    s_endpgm
"""
    v, _ = ring_asm.check(_listing(bad))
    # both the reuse and the next iteration's load into the pending registers
    assert len(v) == 2 and "v_mov_b32 v2, 0" in v[0] and "global_load_dwordx4 v[0:3]" in v[1]
    good = bad.replace("    v_mov_b32 v2, 0\n", "    s_waitcnt vmcnt(0)\n    v_mov_b32 v2, 0\n")
    assert ring_asm.check(_listing(good))[0] == []


def test_decode_ring_is_sound_in_every_e4m3_instance():
    """The check every library build runs: decode.hip compiled to assembly with
    the library's own flags, every all-E4M3 instance (head dims 64/128/256 x
    blocks 16/32) checked."""
    if not shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    build = _load("kvfp8_build_ring", os.path.join("fp8_e4m3_scaled_amd", "build.py"))
    os.makedirs(build.OBJ, exist_ok=True)
    assert build.check_decode_ring() == 6
