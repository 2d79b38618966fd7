"""Host-side checks of the build script: the scan that guards the LM-head
kernel's direct global-to-LDS loads (asm statements that set M0) against any
other use of M0 in that file's assembly."""
from __future__ import annotations

import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _build_module():
    path = os.path.join(HERE, "..", "lossless_speculative_verification_amd", "build.py")
    spec = importlib.util.spec_from_file_location("psispec_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_m0_scan_accepts_the_direct_load_sequence():
    b = _build_module()
    asm = """
_ZN3psi10k_lmh_gemmILi0EEEvNS_6LmhCfgE:
    s_add_i32 s2, s36, s30
    s_mov_b32 m0, s2
    s_nop 0
    global_load_lds_dwordx4 v[90:91], off   ; a load
.LBB1_19:
    v_mfma_f32_32x32x16_bf16 a[32:47], v[58:61], v[82:85], a[32:47]
"""
    assert b.m0_violations(asm) == []


def test_m0_scan_flags_other_uses():
    b = _build_module()
    cases = [
        "s_mov_b32 m0, -1\nds_read_b32 v1, v2\n",                       # the compiler setting M0
        "s_mov_b32 m0, s2\nglobal_load_lds_dwordx4 v[2:3], off\n",       # the wait state missing
        "s_mov_b32 m0, s2\ns_nop 0\nds_write_b32 v1, v2\n",              # M0 feeding something else
        "v_readlane_b32 s4, v1, m0\n",                                   # M0 read
    ]
    for asm in cases:
        assert b.m0_violations(asm), asm
