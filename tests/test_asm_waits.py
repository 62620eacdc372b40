"""Wait states around the hand-scheduled instructions of the head-block attention kernels.

mqa_hb.hip writes some MFMAs and its direct-to-LDS loads as inline assembly, so the compiler
does not insert the wait states the CDNA3/CDNA4 instruction set requires around them; the
source issues them itself and relies on where the compiler places the surrounding code.  This
test compiles the file for gfx950 with the library's own flags and checks the generated
assembly, so that a compiler that places an instruction differently fails here, on the CPU,
and not as wrong numbers on the GPU:

  * a VALU write of a vector register that an inline-assembly MFMA reads as an operand is at
    least 2 wait states ahead of it;
  * no instruction reads or writes an MFMA's result registers within 18 wait states of it (the
    8-pass 32x32x16 bf16 MFMA), except an MFMA that accumulates into exactly those registers;
  * an SGPR written by v_readlane / v_readfirstlane is at least 5 wait states ahead of the
    global_load_lds that reads it.

Wait states are counted one per instruction and N + 1 for s_nop N, within a basic block (a
label or a branch ends the scan; every scan is conservative in that direction).
"""
import os
import re
import shutil
import subprocess

import pytest

from long_context_sparse_15_amd import build as B

SRC = os.path.join(B.SRC, "mqa_hb.hip")


def _hipcc():
    h = B.HIPCC
    return h if h and (os.path.isabs(h) and os.path.exists(h) or shutil.which(h)) else None


@pytest.fixture(scope="module")
def insts(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc is not installed")
    out = str(tmp_path_factory.mktemp("asm") / "mqa_hb.s")
    cmd = ([hipcc] + B.FLAGS + B.FILE_FLAGS.get("mqa_hb.hip", []) +
           ["-I" + B.SRC, "--offload-device-only", "-S", SRC, "-o", out])
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    rows = []  # (kind, text, inside inline assembly)
    in_asm = False
    for line in open(out):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";"):
            continue
        if t.endswith(":") or re.match(r"^[.\w$]+:", t):
            rows.append(("label", t, False))
            continue
        if t.startswith("."):
            continue
        rows.append(("inst", t.split(";")[0].strip(), in_asm))
    return rows


def _regs(tok):
    """The registers a single operand names: v7, a[0:15], s[4:5], ..."""
    tok = tok.strip()
    m = re.match(r"^([vas])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([vas])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(text):
    parts = text.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(",")]


def _ends_block(kind, text):
    return kind == "label" or text.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm"))


def _waits(text):
    if text.startswith("s_nop"):
        return int(text.split()[1], 0) + 1
    return 1


def test_the_kernels_carry_inline_mfmas(insts):
    n = sum(1 for k, t, a in insts if k == "inst" and a and t.startswith("v_mfma"))
    assert n >= 64, "no inline-assembly MFMAs found: the test no longer sees the kernels"


def test_valu_writes_reach_mfma_operands_two_wait_states_ahead(insts):
    bad = []
    for i, (k, t, a) in enumerate(insts):
        if not (k == "inst" and a and t.startswith("v_mfma")):
            continue
        src = set()
        for o in _operands(t)[1:]:
            src |= _regs(o)
        ws, j = 0, i - 1
        while j >= 0 and ws < 2:
            kj, tj, _ = insts[j]
            if _ends_block(kj, tj):
                break
            op = tj.split()[0]
            if (op.startswith("v_") and not op.startswith(("v_mfma", "v_readlane", "v_readfirstlane",
                                                          "v_cmp"))):
                ops = _operands(tj)
                if ops and _regs(ops[0]) & src:
                    bad.append("%s  ->  %s" % (tj, t))
                    break
            ws += _waits(tj)
            j -= 1
    assert not bad, "\n".join(bad[:10])


def test_mfma_results_are_not_touched_before_the_mfma_ends(insts):
    bad = []
    for i, (k, t, a) in enumerate(insts):
        if not (k == "inst" and a and t.startswith("v_mfma")):
            continue
        dst = _regs(_operands(t)[0])
        ws, j = 0, i + 1
        while j < len(insts) and ws < 18:
            kj, tj, _ = insts[j]
            if _ends_block(kj, tj):
                break
            ops = _operands(tj)
            used = set()
            for o in ops:
                used |= _regs(o)
            if tj.startswith("s_nop") or not (used & dst):
                ws += _waits(tj)
                j += 1
                continue
            if (tj.startswith("v_mfma") and len(ops) >= 4 and _regs(ops[0]) == dst and
                    _regs(ops[3]) == dst):
                break  # the next step of the same accumulation (the result is forwarded)
            bad.append("%d wait states: %s  <-  %s" % (ws, tj, t))
            break
    assert not bad, "\n".join(bad[:10])


def test_lds_dma_addresses_are_read_five_wait_states_after_readlane(insts):
    bad = []
    seen = 0
    for i, (k, t, a) in enumerate(insts):
        if not (k == "inst" and t.startswith("global_load_lds")):
            continue
        ops = _operands(t)
        need = set()
        for o in ops[1:]:
            need |= {r for r in _regs(o) if r[0] == "s"}
        if not need:
            continue
        seen += 1
        ws, j = 0, i - 1
        while j >= 0 and ws < 5:
            kj, tj, _ = insts[j]
            if _ends_block(kj, tj):
                break
            if tj.startswith(("v_readlane", "v_readfirstlane")):
                if _regs(_operands(tj)[0]) & need:
                    bad.append("%d wait states: %s  ->  %s" % (ws, tj, t))
                    break
            ws += _waits(tj)
            j -= 1
    assert seen > 0, "no direct-to-LDS loads with a scalar base found"
    assert not bad, "\n".join(bad[:10])
