"""Wait-state checks on the gfx950 assembly of the kernels (CPU only: hipcc
cross-compiles the sources to assembly; nothing runs on a GPU).

The LDS DMA (global_load_lds_dwordx4) and the paired scalar loads of the
attention kernel are written as inline asm, which the compiler's hazard
recognizer does not look inside. These tests hold the generated code to the
GFX9-family rules that matter there:

* a vector memory instruction reads no SGPR that a VALU instruction wrote
  within the previous 5 wait states (a base from v_readfirstlane read too
  early is a stale pointer: an access anywhere in the address space);
* an LDS DMA never directly follows the SALU write of M0 it reads;
* two scalar loads issued back to back inside one asm block never load into
  a register of the other's address.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from bit_sparse_attention_amd import build as B  # noqa: E402

VMEM_SGPR_STATES = 5


def _asm(src: str, tmp_path) -> list[str]:
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"hipcc could not produce assembly for {src}: {r.stderr[-400:]}")
    return out.read_text().split("\n")


def _sregs(tok: str) -> set[int]:
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _instr(line: str) -> str | None:
    t = line.strip()
    if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
        return None
    return t


def _operands(ins: str) -> list[str]:
    parts = ins.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def _lds_dma_violations(lines: list[str]) -> list[str]:
    bad = []
    for i, line in enumerate(lines):
        ins = _instr(line)
        if not ins or not ins.startswith("global_load_lds"):
            continue
        base = _sregs(_operands(ins)[1])
        states, j, first = 0, i - 1, True
        while j >= 0 and states < VMEM_SGPR_STATES:
            p = _instr(lines[j])
            j -= 1
            if p is None:
                continue
            if first and p.startswith("s_mov_b32 m0"):
                bad.append(f"line {i + 1}: LDS DMA directly after the M0 write: {ins}")
            first = False
            m = re.fullmatch(r"s_nop (\d+)", p)
            if m:
                states += int(m.group(1)) + 1
                continue
            if p.startswith("v_") and _sregs(_operands(p)[0] if _operands(p) else "") & base:
                bad.append(f"line {i + 1}: {ins} reads an SGPR written by '{p}' "
                           f"{states} wait states before")
            states += 1
    return bad


def _sload_pair_violations(lines: list[str]) -> list[str]:
    bad = []
    prev = None
    for i, line in enumerate(lines):
        ins = _instr(line)
        if ins is None:
            continue
        if ins.startswith("s_load_dword ") and prev is not None:
            dst = _sregs(_operands(prev)[0])
            addr = _sregs(_operands(ins)[1])
            if dst & addr:
                bad.append(f"line {i + 1}: '{ins}' addresses through the destination of '{prev}'")
        prev = ins if ins.startswith("s_load_dword ") else None
    return bad


@pytest.mark.parametrize("src", ["attn.hip", "linear.hip", "w8a8.hip"])
def test_lds_dma_wait_states(src, tmp_path):
    lines = _asm(src, tmp_path)
    n = sum(1 for l in lines if (_instr(l) or "").startswith("global_load_lds"))
    assert n > 0, f"no LDS DMA found in {src}"
    assert _lds_dma_violations(lines) == []


def test_paired_scalar_loads(tmp_path):
    assert _sload_pair_violations(_asm("attn.hip", tmp_path)) == []


def test_checker_flags_the_hazards():
    """The scanners themselves, on hand-written sequences: a VALU-written base
    2 states before the DMA, M0 written right before it, and a scalar load
    through the previous load's destination are all reported; the padded
    forms are not."""
    hazard = ["v_readfirstlane_b32 s6, v68", "v_and_or_b32 v69, v69, s2, v71",
              "s_mov_b32 m0, s3", "global_load_lds_dwordx4 v69, s[6:7]"]
    found = _lds_dma_violations(hazard)
    assert any("wait states before" in b for b in found)
    assert any("directly after the M0 write" in b for b in found)
    padded = ["v_readfirstlane_b32 s6, v68", "v_and_or_b32 v69, v69, s2, v71",
              "s_mov_b32 m0, s3", "s_nop 3", "global_load_lds_dwordx4 v69, s[6:7]"]
    assert _lds_dma_violations(padded) == []
    assert _sload_pair_violations(["s_load_dword s6, s[2:3], 0x0", "s_load_dword s4, s[6:7], 0x0"])
    assert not _sload_pair_violations(["s_load_dword s6, s[2:3], 0x0",
                                       "s_load_dword s4, s[8:9], 0x0"])
