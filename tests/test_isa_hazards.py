"""Matrix-core result spacing in the compiled gfx950 code.

A value produced by a v_mfma instruction may be read only after a number of
independent wait states; on CDNA the hardware does not interlock these reads,
so a read that comes too early silently takes a stale accumulator.  The
compiler inserts the spacing itself, but a path through a conditional branch
once reached such a read after two wait states (the compose kernel then lost
one accumulator register's contribution).  This test compiles every kernel
source to assembly and walks the control-flow graph of each kernel: on every
path from a matrix-core instruction to an instruction that reads any of its
destination registers there must be at least MIN_WAIT[opcode] wait states
(one per instruction, n + 1 per s_nop n): the spacing the compiler itself
keeps on straight-line code, 8 after the 16x16x32 and 16x16x16
half-precision (fp16 and bf16) products, 12 after the 32x32x16 fp16 product and
10 after the 8-pass 16x16x4 fp32 product.  A matrix-core opcode
without a figure here fails the test, so a new one gets a deliberate entry.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from state_caching_amd import build as hb

MIN_WAIT = {
    "v_mfma_f32_16x16x32_bf16": 8,
    "v_mfma_f32_16x16x32_f16": 8,
    "v_mfma_f32_16x16x16_f16": 8,
    "v_mfma_f32_16x16x16_bf16": 8,
    "v_mfma_f32_32x32x16_f16": 12,
    "v_mfma_f32_16x16x4_f32": 10,
}
_REG = re.compile(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _functions(asm: str) -> dict:
    funcs, cur = {}, None
    for line in asm.splitlines():
        t = line.split(";")[0].strip()
        m = re.match(r"^(_Z\w+):", t)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None or not t:
            continue
        if t.startswith(".") and not t.endswith(":"):
            if t.startswith(".Lfunc_end"):
                cur = None
            continue
        funcs[cur].append(t)
    return funcs


def short_paths(lines: list) -> list:
    """(mfma index, reader index, wait states) for every too-early read."""
    ins, labels = [], {}
    for t in lines:
        if t.endswith(":"):
            labels[t[:-1]] = len(ins)
        else:
            ins.append(t)

    def succ(i):
        op = ins[i].split()[0]
        if op == "s_endpgm":
            return []
        if op == "s_branch":
            return [labels[ins[i].split()[1]]]
        out = [labels[ins[i].split()[1]]] if op.startswith("s_cbranch") else []
        if i + 1 < len(ins):
            out.append(i + 1)
        return out

    found = []
    for i, t in enumerate(ins):
        op = t.split()[0]
        if not op.startswith("v_mfma"):
            continue
        need = MIN_WAIT.get(op)
        if need is None:
            found.append((i, i, -1))
            continue
        dst = _regs(t[len(op):].split(",")[0])
        stack, seen = [(j, 0) for j in succ(i)], set()
        while stack:
            j, w = stack.pop()
            if w >= need or (j, w) in seen:
                continue
            seen.add((j, w))
            tj = ins[j]
            opj = tj.split()[0]
            args = tj[len(opj):].split(",")
            if opj == "s_nop":
                for k in succ(j):
                    stack.append((k, w + int(tj.split()[1], 0) + 1))
                continue
            if opj.startswith("v_mfma"):
                # a chained accumulator (srcC) is forwarded by the hardware
                src = set().union(*[_regs(a) for a in args[1:3]])
            elif opj.startswith(("ds_write", "global_store", "buffer_store")):
                src = set().union(*[_regs(a) for a in args])
            else:
                src = set().union(*[_regs(a) for a in args[1:]]) if len(args) > 1 else set()
            if dst & src:
                found.append((i, j, w))
                continue
            for k in succ(j):
                stack.append((k, w + 1))
    return found


def test_scanner_flags_a_branch_path():
    # the shape that went wrong: the read sits right behind a taken branch
    lines = [
        "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[4:7], a[4:7]",
        "s_cbranch_scc0 .L1",
        "v_mov_b32 v9, 0", "v_mov_b32 v9, 0", "v_mov_b32 v9, 0", "v_mov_b32 v9, 0",
        "v_mov_b32 v9, 0", "v_mov_b32 v9, 0", "v_mov_b32 v9, 0", "v_mov_b32 v9, 0",
        ".L1:",
        "v_accvgpr_read_b32 v10, a7",
        "s_endpgm",
    ]
    assert short_paths(lines) == [(0, 10, 1)]
    padded = lines[:1] + ["s_nop 7"] + lines[1:]
    assert short_paths(padded) == []
    # the 8-pass fp32 product needs more room than the s_nop 7 above gives
    f32 = [padded[0].replace("16x16x32_bf16", "16x16x4_f32")] + padded[1:]
    assert short_paths(f32) == [(0, 11, 9)]
    unknown = [padded[0].replace("16x16x32_bf16", "32x32x16_bf16")] + padded[1:]
    assert short_paths(unknown) == [(0, 0, -1)]


def _asm(src: str) -> str:
    out = os.path.join(hb.BUILD_DIR, "isa_" + os.path.splitext(src)[0] + ".s")
    cmd = [hb.HIPCC, *hb.FLAGS, "--cuda-device-only", "-S", os.path.join(hb.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"hipcc -S failed on {src}:\n{r.stderr[-2000:]}")
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(not os.path.exists(hb.HIPCC), reason="hipcc not available")
def test_kernel_mfma_result_spacing():
    os.makedirs(hb.BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, len(hb.SOURCES))) as ex:
        texts = dict(zip(hb.SOURCES, ex.map(_asm, hb.SOURCES)))
    bad = []
    for src, asm in texts.items():
        for fn, lines in _functions(asm).items():
            for i, j, w in short_paths(lines):
                bad.append(f"{src} {fn}: mfma #{i} read by #{j} after {w} wait states"
                           if w >= 0 else f"{src} {fn}: no spacing figure for mfma #{i}")
    assert not bad, "\n".join(bad[:20])
