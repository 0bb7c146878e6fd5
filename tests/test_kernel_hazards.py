"""Wait states around the hand-written MFMAs (CPU only: hipcc cross-compiles).

The bf16 main loop issues its MFMAs from inline assembly, so that each one
accumulates in place.  The compiler does not know such an instruction is an
MFMA and inserts none of the wait states the hardware needs around one:
  * an MFMA reads its A and B operands a few cycles after issue, so a VALU
    write of one of them needs independent instructions before the MFMA;
  * an MFMA writes its result many cycles after issue, so any other
    instruction that reads or overwrites the result registers must wait.
The kernels provide both by construction (operands come from LDS reads, the
main loop ends in 32 wait states and an in-place fence of the accumulators).
This test compiles kernels.hip to assembly and checks every path the
compiler could have broken: no VALU write of an MFMA operand within 2 wait
states before it, and no access to an MFMA's result registers other than by
another MFMA within 20 wait states after it (the longest bf16 MFMA needs
fewer).  Paths follow fall-through and loop back-edges; a label right after
an unconditional branch starts a new path."""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from grpo_policy_loss_amd import build as libbuild

VALU_BEFORE = 2     # wait states a VALU write of an operand needs before the MFMA
RESULT_AFTER = 20   # wait states before another instruction may touch the result


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(ins):
    return [t.strip() for t in ins.split(None, 1)[1].split(",")] if " " in ins else []


def _wait_states(ins):
    return int(ins.split()[1]) + 1 if ins.startswith("s_nop") else 1


def _functions(asm):
    """{name: [(kind, text)]} with kind 'ins', 'asm-mfma' or 'label'."""
    funcs, cur, in_asm = {}, None, False
    for line in asm.split("\n"):
        s = line.strip()
        m = re.match(r"^(_Z[\w$]+):(\s|$)", line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif re.match(r"^\.LBB\d+_\d+:", s):
            cur.append(("label", s.split(":")[0]))
        elif s and not s.startswith((";", ".")):
            kind = "asm-mfma" if in_asm and s.startswith("v_mfma") else "ins"
            cur.append((kind, s.split(";")[0].strip()))
    return funcs


def _paths(items):
    """Straight-line instruction sequences: fall-through runs, plus each loop
    back-edge's tail joined to its header."""
    runs, run = [], []
    for k, (kind, text) in enumerate(items):
        if kind == "label":
            prev = run[-1][1] if run else ""
            if prev.startswith(("s_branch", "s_endpgm", "s_setpc")):
                runs.append(run)
                run = []
            continue
        run.append((kind, text))
    runs.append(run)
    labels = {text: k for k, (kind, text) in enumerate(items) if kind == "label"}
    for k, (kind, text) in enumerate(items):
        m = re.match(r"s_(c?branch\w*)\s+(\.LBB\d+_\d+)$", text) if kind == "ins" else None
        if m and labels.get(m.group(2), k) < k:
            head = [x for x in items[labels[m.group(2)]:labels[m.group(2)] + 200] if x[0] != "label"]
            tail = [x for x in items[max(0, k - 200):k + 1] if x[0] != "label"]
            runs.append(tail + head)
    return runs


def _violations(seq):
    bad = []
    for k, (kind, text) in enumerate(seq):
        if kind == "asm-mfma":
            srcs = set().union(set(), *(_regs(o) for o in _operands(text)[1:4]))
            ws = 0
            for b in range(k - 1, -1, -1):
                pk, pt = seq[b]
                ws += _wait_states(pt)
                if ws > VALU_BEFORE:
                    break
                if pk == "ins" and pt.startswith("v_") and " " in pt:
                    if _regs(_operands(pt)[0]) & srcs:
                        bad.append(f"VALU write {pt!r} {ws} wait state(s) before {text!r}")
            continue
        if text.startswith("v_mfma"):
            continue            # MFMAs order among themselves
        touched = set().union(set(), *(_regs(o) for o in _operands(text)))
        if not touched:
            continue
        ws = 0
        for b in range(k - 1, -1, -1):
            pk, pt = seq[b]
            ws += _wait_states(pt)
            if ws >= RESULT_AFTER:
                break
            if pk == "asm-mfma" and _regs(_operands(pt)[0]) & touched:
                bad.append(f"{text!r} {ws} wait state(s) after {pt!r}")
                break
    return bad


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    try:
        hipcc = libbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    cmd = [hipcc, *libbuild.HIPCC_FLAGS, "--cuda-device-only", "-S",
           os.path.join(libbuild.CSRC, "kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_the_scan_finds_both_kinds_of_hazard():
    seq = [("ins", "v_accvgpr_read_b32 v20, a180"),
           ("asm-mfma", "v_mfma_f32_16x16x32_bf16 a[0:3], v[16:19], v[20:23], a[0:3]"),
           ("ins", "s_nop 0"),
           ("ins", "v_accvgpr_read_b32 v30, a2")]
    bad = _violations(seq)
    assert len(bad) == 2 and "before" in bad[0] and "after" in bad[1]
    fine = [("ins", "v_accvgpr_read_b32 v20, a180"), ("ins", "s_nop 1"),
            ("asm-mfma", "v_mfma_f32_16x16x32_bf16 a[0:3], v[16:19], v[20:23], a[0:3]"),
            ("ins", "s_nop 7"), ("ins", "s_nop 7"), ("ins", "s_nop 7"),
            ("ins", "v_accvgpr_read_b32 v30, a2")]
    assert _violations(fine) == []


def test_no_wait_state_hazards_around_the_inline_mfmas(assembly):
    funcs = _functions(assembly)
    with_asm = {n: f for n, f in funcs.items() if any(k == "asm-mfma" for k, _ in f)}
    assert with_asm, "no inline-assembly MFMA found"
    problems = []
    for name, items in with_asm.items():
        for seq in _paths(items):
            problems += [f"{name[:60]}: {p}" for p in _violations(seq)]
    assert not problems, "\n".join(problems[:20])
