"""Checks on the generated gfx950 code of the attention kernels (CPU only:
hipcc cross-compiles)."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Instructions that name M0, or read or write it without naming it: GPR
# indexing (s_set_gpr_idx_on, s_movrel*, v_movrel*), messages, GWS,
# interpolation and the LDS-DMA loads.
M0_USE = re.compile(r"\bm0\b|s_set_gpr_idx|movrel|s_sendmsg|ds_gws|v_interp|load_lds|_lds_dword")


def m0_uses(asm_lines):
    """(uses inside inline-asm blocks, [(line, text) of uses outside them])."""
    in_asm, ours, stray = False, 0, []
    for n, line in enumerate(asm_lines, 1):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif s and not s.startswith((";", ".")) and M0_USE.search(s):
            if in_asm:
                ours += 1
            else:
                stray.append((n, s))
    return ours, stray


def test_m0_is_used_only_by_the_lds_loads(tmp_path):
    """The tile and page-table loads (global_load_lds) take their LDS
    destination from M0, which they set in inline asm and list as clobbered.
    The compiler reserves M0 and does not restore a value of its own around
    such asm, so the kernels must not rely on one: outside those asm blocks
    the generated code reads or writes M0 nowhere (also not implicitly, as
    GPR indexing does)."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    sys.path.insert(0, ROOT)
    from mla_absorbed_tree_amd import build_lib
    src = os.path.join(ROOT, "mla_absorbed_tree_amd", "csrc", "verify_attn.hip")
    out = tmp_path / "verify_attn.s"
    flags = [f for f in build_lib.HIP_FLAGS if not f.startswith("-W")]
    subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", src, "-o", str(out)], check=True,
                   capture_output=True)
    ours, stray = m0_uses(open(out))
    assert ours > 0, "no M0 write found in the load asm (did the loads change?)"
    assert not stray, stray[:5]


def test_m0_check_sees_implicit_uses():
    """The check flags M0 uses the compiler makes without naming the register
    (dynamic register indexing), and counts the asm blocks' own."""
    sample = [
        "\ts_mov_b32 s2, 3",
        "\ts_set_gpr_idx_on s2, gpr_idx(SRC0)",
        "\tv_mov_b32_e32 v0, v1",
        "\ts_set_gpr_idx_off",
        "\t;;#ASMSTART",
        "\ts_mov_b32 m0, s4",
        "\tglobal_load_lds_dwordx4 v[2:3], off",
        "\t;;#ASMEND",
        "\tds_read_b128 v[4:7], v8",
    ]
    ours, stray = m0_uses(sample)
    assert ours == 2 and [n for n, _ in stray] == [2, 4]
