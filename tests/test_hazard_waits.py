"""Wait states around matrix (MFMA) instructions in the compiled decode kernels (CPU test).

The row-owner decode kernel issues its MFMAs as inline asm (its output accumulators live in
the AGPRs, which the compiler would otherwise route through VGPRs).  The compiler inserts no
hazard waits around inline asm, so each asm group carries its own: two wait states before an
MFMA whose operands a vector-ALU instruction may have just written, and a drain after the
last MFMA of a phase before anything else reads or overwrites its results.  This test
compiles the kernels to gfx950 assembly with the build's own flags and checks, along every
path of the control-flow graph, the CDNA3/CDNA4 rules:

  * a VALU write of a VGPR or AGPR is followed by at least 2 wait states before an MFMA
    reads it (as A, B or C operand);
  * an MFMA's result registers are not read or written by a non-MFMA instruction, nor read as
    an A/B operand by another MFMA, within passes + 4 wait states (8 for the 4-pass
    16x16x32 bf16 MFMA, the count the compiler itself inserts after its own MFMAs);
  * back-to-back accumulation (an MFMA of the same shape takes the result, exactly
    overlapped, as its C operand) needs no wait, and one MFMA overwriting another's result
    is ordered by the matrix pipe (the compiler itself issues such pairs 4 states apart).

A wait state is one issued instruction; ``s_nop N`` provides N + 1.  Meta lines (labels,
comments, directives) provide none.  The compiler-generated MFMAs of the other decode kernels
are checked too: they show the checker agrees with the compiler's own hazard handling.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from mla_latent_kv_02_amd import build as libbuild

KERNEL_FILES = ["mla_decode_rows.hip", "mla_decode.hip"]
VALU_TO_MFMA = 2
# passes of 4 cycles each (16x16x32 bf16: 16 cycles); unknown shapes are taken as 16 passes
PASSES = {"16x16x32": 4, "32x32x16": 8}

REG = re.compile(r"\b([va])(?:(\d+)|\[(\d+):(\d+)\])")


def regs(tok: str):
    """Set of ('v'|'a', index) named by one operand token."""
    out = set()
    for m in REG.finditer(tok):
        kind = m.group(1)
        if m.group(2) is not None:
            out.add((kind, int(m.group(2))))
        else:
            out.update((kind, i) for i in range(int(m.group(3)), int(m.group(4)) + 1))
    return out


class Inst:
    def __init__(self, text: str):
        self.text = text
        parts = text.split(None, 1)
        self.op = parts[0]
        self.ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        self.is_mfma = self.op.startswith("v_mfma")
        self.is_nop = self.op == "s_nop"
        self.waits = int(self.ops[0], 0) + 1 if self.is_nop else 1
        self.branch_target = None
        if self.op.startswith("s_cbranch") or self.op == "s_branch":
            self.branch_target = self.ops[0] if self.ops else None
        self.unconditional = self.op in ("s_branch", "s_endpgm", "s_setpc_b64")
        # destination / sources
        self.dst, self.src = set(), set()
        if self.is_mfma:
            self.dst = regs(self.ops[0])
            self.src_ab = regs(self.ops[1]) | regs(self.ops[2])
            self.src_c = regs(self.ops[3]) if len(self.ops) > 3 else set()
            self.src = self.src_ab | self.src_c
            m = re.search(r"(\d+x\d+x\d+)", self.op)
            self.passes = PASSES.get(m.group(1), 16) if m else 16
        elif self.op.startswith("v_") or self.op.startswith("ds_read") or self.op.startswith("global_load") \
                or self.op.startswith("buffer_load") or self.op.startswith("flat_load") or self.op.startswith("scratch_load"):
            if self.ops:
                self.dst = regs(self.ops[0])
            self.src = set().union(*(regs(o) for o in self.ops[1:])) if len(self.ops) > 1 else set()
        else:
            self.src = set().union(*(regs(o) for o in self.ops)) if self.ops else set()
        self.is_valu = self.op.startswith("v_") and not self.is_mfma


def parse_functions(asm: str):
    """{kernel name: (instructions, {label: index})} of every function in the assembly."""
    funcs = {}
    cur = None
    for raw in asm.splitlines():
        line = raw.split(";")[0].rstrip()
        m = re.match(r"^([_A-Za-z.$][\w.$]*):", line)
        if m and not line.startswith("\t"):
            name = m.group(1)
            if not name.startswith(".L") and not name.startswith("$"):
                cur = funcs.setdefault(name, ([], {}))
                continue
            if cur is not None:
                cur[1][name] = len(cur[0])
            continue
        if cur is None:
            continue
        s = line.strip()
        if not s or s.startswith("."):
            if s.startswith(".Lfunc_end") or s.startswith(".end_amdhsa"):
                cur = None
            continue
        cur[0].append(Inst(s))
    return funcs


def successors(insts, labels, i):
    """Indices that can execute right after instruction i."""
    ins = insts[i]
    out = []
    if ins.branch_target is not None and ins.branch_target in labels:
        out.append(labels[ins.branch_target])
    if not ins.unconditional and i + 1 < len(insts):
        out.append(i + 1)
    return out


def predecessors(insts, labels):
    pred = {i: [] for i in range(len(insts))}
    for i in range(len(insts)):
        for j in successors(insts, labels, i):
            pred[j].append(i)
    return pred


def check(insts, labels):
    """List of violations (strings)."""
    bad = []
    pred = predecessors(insts, labels)
    for i, ins in enumerate(insts):
        if not ins.is_mfma:
            continue
        # backwards: VALU writes of this MFMA's operands within VALU_TO_MFMA wait states
        stack = [(p, 0) for p in pred[i]]
        seen = set()
        while stack:
            j, w = stack.pop()
            if (j, w) in seen or w >= VALU_TO_MFMA:
                continue
            seen.add((j, w))
            pj = insts[j]
            if pj.is_valu and pj.dst & ins.src:
                bad.append(f"VALU '{pj.text}' writes an operand of '{ins.text}' {w} wait states before it")
            stack.extend((p, w + pj.waits) for p in pred[j])
        # forwards: readers and writers of the result within passes + 4 wait states
        need = ins.passes + 4
        stack = [(s, 0) for s in successors(insts, labels, i)]
        seen = set()
        while stack:
            j, w = stack.pop()
            if (j, w) in seen or w >= need:
                continue
            seen.add((j, w))
            nj = insts[j]
            if nj.is_mfma:
                # the result taken whole as the C operand of an MFMA of the same shape is forwarded
                chained = nj.op == ins.op and nj.src_c == ins.dst
                if nj.src_ab & ins.dst or (nj.src_c & ins.dst and not chained):
                    bad.append(f"'{nj.text}' reads the result of '{ins.text}' {w} wait states after it")
                if chained and nj.dst == ins.dst:
                    continue   # the chain's next MFMA carries the dependency on
            elif (nj.src | nj.dst) & ins.dst:
                bad.append(f"'{nj.text}' touches the result of '{ins.text}' {w} wait states after it")
            stack.extend((s, w + nj.waits) for s in successors(insts, labels, j))
    return bad


@pytest.fixture(scope="module")
def assembly():
    hipcc = libbuild._hipcc()
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        for f in KERNEL_FILES:
            dst = os.path.join(tmp, f + ".s")
            cmd = [hipcc] + libbuild.COMMON + ["--cuda-device-only", "-S", os.path.join(libbuild.CSRC, f), "-o", dst]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            out[f] = open(dst).read()
    return out


@pytest.mark.parametrize("fname", KERNEL_FILES)
def test_mfma_wait_states(assembly, fname):
    funcs = parse_functions(assembly[fname])
    kernels = {k: v for k, v in funcs.items() if "decode" in k}
    assert kernels, "no decode kernel found in the assembly"
    n_mfma = 0
    problems = []
    for name, (insts, labels) in kernels.items():
        n_mfma += sum(1 for x in insts if x.is_mfma)
        problems += [f"{name}: {p}" for p in check(insts, labels)]
    assert n_mfma > 0
    assert not problems, "\n".join(problems[:20])


def test_checker_catches_missing_waits():
    """The checker itself: a VALU write right before an MFMA, and a read of an MFMA result
    without a drain, are flagged; the same code with the waits is clean."""
    def run(lines):
        insts = [Inst(x) for x in lines]
        return check(insts, {})
    bad_pre = ["v_mov_b32 v4, 0", "v_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[4:7], 0", "s_nop 7", "s_nop 7",
               "s_endpgm"]
    assert run(bad_pre)
    ok_pre = ["v_mov_b32 v4, 0", "s_nop 1", "v_mfma_f32_16x16x32_bf16 v[8:11], v[0:3], v[4:7], 0", "s_nop 7",
              "s_nop 7", "s_endpgm"]
    assert not run(ok_pre)
    bad_post = ["v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", "s_nop 5",
                "global_store_dwordx4 v20, a[0:3], off", "s_endpgm"]
    assert run(bad_post)
    ok_post = ["v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
               "v_mfma_f32_16x16x32_bf16 a[0:3], v[12:15], v[4:7], a[0:3]", "s_nop 7", "s_nop 3",
               "global_store_dwordx4 v20, a[0:3], off", "s_endpgm"]
    assert not run(ok_post)
