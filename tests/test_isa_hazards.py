"""Wait-state check of the hand-written global->LDS copies in the built device code.

The copies are inline asm (`dma16`), and the compiler does not resolve hazards for
instructions inside inline asm. On gfx9-family chips a vector-memory instruction
needs 5 wait states after a VALU instruction writes an SGPR that it reads (its
base address), and an LDS-DMA load needs 1 wait state after a scalar write of M0
(its LDS address). This test compiles every HIP source that issues such a copy to
gfx950 assembly with the library's own flags and checks, for every LDS-DMA load,
that the instructions in front of it inside its basic block give those wait
states. It also checks the scanner on hand-written snippets with planted hazards.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_sparse_global_mean_amd import build as B

VMEM_SGPR_WAIT = 5
M0_WAIT = 1


def _sregs(tok: str) -> set:
    tok = tok.strip()
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _instructions(asm: str):
    """(line number, text) per instruction; 'LABEL' marks a basic-block boundary."""
    out = []
    for i, line in enumerate(asm.splitlines(), 1):
        t = line.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":"):
            out.append((i, "LABEL"))
        elif t.startswith("."):
            continue
        else:
            out.append((i, t))
    return out


def _wait_states(t: str) -> int:
    m = re.match(r"s_nop\s+(\d+)", t)
    return int(m.group(1)) + 1 if m else 1


def lds_dma_hazards(asm: str) -> list:
    """Problems found in front of each global_load_lds* instruction of `asm`."""
    ins = _instructions(asm)
    problems = []
    for k, (line, t) in enumerate(ins):
        if not t.startswith("global_load_lds"):
            continue
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        base = _sregs(ops[1]) if len(ops) > 1 else set()
        ws, j = 0, k - 1
        while ws < VMEM_SGPR_WAIT:
            if j < 0 or ins[j][1] == "LABEL":
                problems.append((line, t, f"block starts {ws} wait states before"))
                break
            tj = ins[j][1]
            op = tj.split()[0]
            args = [a.strip() for a in tj.split(None, 1)[1].split(",")] if " " in tj else []
            if ws < M0_WAIT and op.startswith("s_") and args and args[0] == "m0":
                problems.append((line, t, f"M0 written {ws} wait states before by {tj}"))
            if op.startswith("v_") and args:
                written = _sregs(args[0])
                if op.startswith(("v_add_co", "v_sub_co", "v_addc", "v_subb", "v_mad_u64", "v_mad_i64",
                                  "v_div_scale")) and len(args) > 1:
                    written |= _sregs(args[1])
                if written & base:
                    problems.append((line, t, f"base written {ws} wait states before by {tj}"))
            ws += _wait_states(tj)
            j -= 1
    return problems


def test_scanner_finds_planted_hazards():
    ok = """
.LBB0_1:
    v_readfirstlane_b32 s4, v2
    s_add_i32 s7, s7, 1
    s_mov_b32 m0, s3
    s_nop 4
    global_load_lds_dwordx4 v9, s[4:5]
"""
    assert lds_dma_hazards(ok) == []
    valu = ok.replace("s_nop 4\n", "s_nop 1\n")
    found = lds_dma_hazards(valu)
    assert len(found) == 1 and "base written 4 wait states" in found[0][2]
    m0 = ok.replace("    s_nop 4\n", "").replace("s_mov_b32 m0, s3", "s_nop 4\n    s_mov_b32 m0, s3")
    assert any("M0 written 0" in p[2] for p in lds_dma_hazards(m0))
    short_block = ".LBB0_2:\n    s_nop 2\n    global_load_lds_dwordx4 v9, s[4:5]\n"
    assert "block starts 3" in lds_dma_hazards(short_block)[0][2]
    spill = ok.replace("s_add_i32 s7, s7, 1", "v_readlane_b32 s5, v255, 3")
    assert lds_dma_hazards(spill) == []          # 5 wait states from the nop alone
    assert lds_dma_hazards(spill.replace("s_nop 4", "s_nop 0"))


def _sources_with_lds_dma():
    out = []
    for src in B.SOURCES:
        text = open(os.path.join(B.CSRC, src)).read()
        if "dma16(" in text or "global_load_lds" in text:
            out.append(src)
    return out


def _device_asm(src: str, tmp) -> str:
    path = os.path.join(str(tmp), os.path.splitext(src)[0] + ".s")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return open(path).read()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_built_copies_have_their_wait_states(tmp_path):
    srcs = _sources_with_lds_dma()
    assert "attn_bf16.hip" in srcs and "dense_rows.hip" in srcs
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        asms = list(ex.map(lambda s: _device_asm(s, tmp_path), srcs))
    for src, asm in zip(srcs, asms):
        n = sum(1 for _, t in _instructions(asm) if t.startswith("global_load_lds"))
        assert n > 0, f"{src}: no LDS-DMA loads found in the assembly"
        problems = lds_dma_hazards(asm)
        assert not problems, f"{src}: " + "; ".join(f"line {l}: {p}" for l, _, p in problems[:5])
