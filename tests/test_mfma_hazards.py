"""Hazards of the MLA kernel's score products, checked on the gfx950 assembly the library is built from.

The score products of mla32_kernel are written in inline assembly in their VGPR-accumulator form (the output
accumulators fill the AGPR file), and the compiler does not track hazards through inline assembly.  Its own
code around them must therefore keep two distances, which this test checks in the emitted assembly of both
template instances:
  - after a product that writes VGPRs, nothing reads or writes those registers for 20 wait states, except
    the next product of the same chain, which takes them whole as its accumulator (forwarded in hardware);
  - before a product, no VALU instruction writes one of its operands within 2 wait states.
The check follows the listing's control flow (fall-through and branch targets), forward from every product
and backward into it.  Planted listings show that it catches both kinds, on a taken branch too, and that it
does not follow an unconditional branch's fall-through.
"""
import os
import re
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = ["_ZN3hsk12mla32_kernelILi4EEEvNS_7MlaArgsE", "_ZN3hsk12mla32_kernelILi2EEEvNS_7MlaArgsE"]
AFTER, BEFORE = 20, 2
_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(op):
    out = set()
    for m in _REG.finditer(op):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _parse(lines):
    """Instructions as (op, text, args); a label is ("LABEL", name, [])."""
    ins = []
    for ln in lines:
        t = ln.split(";")[0].strip()
        if not t or t.startswith("."):
            if t.startswith(".LBB") and t.endswith(":"):
                ins.append(("LABEL", t[:-1], []))
            continue
        if t.endswith(":"):
            continue
        parts = t.split(None, 1)
        args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        ins.append((parts[0], t, args))
    return ins


def _wait_states(op, args):
    if op == "LABEL":
        return 0
    return int(args[0], 0) + 1 if op == "s_nop" else 1


def _cfg(ins):
    """Successors of every instruction: fall-through, branch targets (both for a conditional branch)."""
    label = {t: i for i, (op, t, _) in enumerate(ins) if op == "LABEL"}
    succ = []
    for i, (op, t, args) in enumerate(ins):
        nxt = [i + 1] if i + 1 < len(ins) else []
        if op == "s_branch":
            succ.append([label[args[0]]] if args[0] in label else [])
        elif op.startswith("s_cbranch"):
            succ.append(nxt + ([label[args[0]]] if args and args[0] in label else []))
        elif op == "s_endpgm":
            succ.append([])
        else:
            succ.append(nxt)
    pred = [[] for _ in ins]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].append(i)
    return succ, pred


def hazards(ins):
    """(kind, product, offending instruction) for every violation on any path of a parsed listing."""
    succ, pred = _cfg(ins)
    bad = []
    for k, (op, t, args) in enumerate(ins):
        if not op.startswith("v_mfma") or not args[0].startswith("v"):
            continue
        dst = _regs(args[0])
        # forward: along every path, nothing touches dst within AFTER wait states, except a chained product
        # accumulating into exactly dst (which then carries the check on)
        stack, seen = [(j, 0) for j in succ[k]], set()
        while stack:
            i, ws = stack.pop()
            if (i, ws) in seen or ws >= AFTER:
                continue
            seen.add((i, ws))
            op2, t2, a2 = ins[i]
            touched = set().union(*(_regs(a) for a in a2)) if (a2 and op2 != "s_nop") else set()
            if touched & dst:
                chained = op2.startswith("v_mfma") and len(a2) > 3 and a2[3] == args[0] \
                    and not (_regs(a2[1]) | _regs(a2[2])) & dst
                if not chained:
                    bad.append(("after", t, t2))
                continue
            stack.extend((j, ws + _wait_states(op2, a2)) for j in succ[i])
        # backward: along every path into the product, no VALU write of an operand within BEFORE wait states
        srcs = set().union(*(_regs(a) for a in args[1:4]))
        stack, seen = [(j, 0) for j in pred[k]], set()
        while stack:
            i, ws = stack.pop()
            if (i, ws) in seen or ws >= BEFORE:
                continue
            seen.add((i, ws))
            op2, t2, a2 = ins[i]
            if op2.startswith("v_") and not op2.startswith("v_mfma") and a2 and _regs(a2[0]) & srcs:
                bad.append(("before", t, t2))
                continue
            stack.extend((j, ws + _wait_states(op2, a2)) for j in pred[i])
    return bad


def _kernel(lines, name):
    start = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    return _parse(lines[start:end + 1])


def test_checker_follows_branches():
    """A write reached only by a branch is checked on that path; one behind an unconditional branch is not on the
    fall-through path."""
    taken = """
        v_mfma_f32_32x32x16_bf16 v[18:33], v[10:13], v[162:165], 0
        s_cbranch_vccnz .LBB0_2
        s_nop 7
        s_nop 7
        s_nop 7
    .LBB0_2:
        v_mov_b32_e32 v20, 0
        s_endpgm
    """.strip().split("\n")
    assert [b[0] for b in hazards(_parse(taken))] == ["after"]
    skipped = """
        v_mfma_f32_32x32x16_bf16 v[18:33], v[10:13], v[162:165], 0
        s_branch .LBB0_3
    .LBB0_2:
        v_mov_b32_e32 v20, 0
    .LBB0_3:
        s_nop 7
        s_nop 7
        s_nop 7
        v_mov_b32_e32 v21, 0
        s_endpgm
    """.strip().split("\n")
    assert hazards(_parse(skipped)) == []


def test_checker_catches_planted_hazards():
    listing = """
        v_mfma_f32_32x32x16_bf16 v[18:33], v[10:13], v[162:165], 0
        v_mfma_f32_32x32x16_bf16 v[18:33], v[2:5], v[166:169], v[18:33]
        s_nop 0
        v_mov_b64_e32 v[2:3], v[18:19]
        v_mov_b32_e32 v170, 0
        v_mfma_f32_32x32x16_bf16 v[40:55], v[6:9], v[170:173], v[18:33]
        s_nop 7
        s_nop 7
        s_nop 3
        v_add_f32_e32 v1, v40, v41
    """.strip().split("\n")
    bad = hazards(_parse(listing))
    assert [b[0] for b in bad] == ["after", "before"], bad
    assert "v_mov_b64_e32 v[2:3], v[18:19]" in bad[0][2] and "v_mov_b32_e32 v170, 0" in bad[1][2]
    # the same listing with the copy and the write moved out of reach is clean
    fixed = [l for l in listing if "v_mov" not in l]
    assert hazards(_parse(fixed)) == []


@pytest.mark.skipif(not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")), reason="needs hipcc")
def test_mla32_score_products_keep_their_distances(tmp_path):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "hsk_build", os.path.join(ROOT, "hierarchical_sparse_kv_layer_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    out = str(tmp_path / "attention.s")
    b.device_asm("attention.hip", out)
    lines = open(out).read().split("\n")
    for name in KERNELS:
        ins = _kernel(lines, name)
        n_vgpr_form = sum(1 for op, _, a in ins if op.startswith("v_mfma") and a[0].startswith("v"))
        assert n_vgpr_form >= 36, (name, n_vgpr_form)     # at least one full score chain
        bad = hazards(ins)
        assert bad == [], (name, bad[:5])
        print(f"{name}: {n_vgpr_form} VGPR-form products, no hazard", file=sys.stderr)
