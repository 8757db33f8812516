"""Static checks of the built gfx950 code (no GPU): the device assembly of the
HIP sources is scanned for two code-generation hazards.

* Store data: a VALU write to a data register of a store wider than 8 bytes,
  issued directly behind the store, has reached memory in place of the stored
  value on gfx950 for some lanes, and the compiler inserts no wait state
  there.  No such pair may appear.
* Inline-asm LDS reads: the compiler takes an asm read's destination as
  written when the asm issues, although the data lands only at the matching
  s_waitcnt lgkmcnt.  On every path from such a read to the next
  `s_waitcnt lgkmcnt(0)`, no instruction may touch its destination registers.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "loss_head_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
from loss_head_amd.build import SOURCES  # noqa: E402  (every source the library is built from)
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wno-unused-result", "--cuda-device-only", "-S"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa")
    out = {}
    for src in SOURCES:
        dst = str(d / src.replace(".hip", ".s"))
        p = subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", dst], capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-2000:]
        out[src] = open(dst).read()
    return out


def _regs(tok):
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _functions(text):
    """(name, [(instruction, inside inline asm)], {label: index})."""
    for m in re.finditer(r"^([A-Za-z_][\w.$]*):\s*(;.*)?$", text, re.M):
        name = m.group(1)
        if name.startswith(".") or not name.startswith("_Z"):
            continue
        end = text.find(".Lfunc_end", m.end())
        ins, labels, in_asm = [], {}, False
        for line in text[m.end():end].splitlines():
            t = line.strip()
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not t or t.startswith(";") or t.startswith("."):
                lab = re.match(r"^(\.LBB\w+):", t)
                if lab:
                    labels[lab.group(1)] = len(ins)
                continue
            ins.append((t.split(";")[0].strip(), in_asm))
        yield name, ins, labels


def _operands(t):
    op = t.split()[0]
    return op, [o.strip() for o in t[len(op):].split(",")]


WIDE_STORE = re.compile(r"^(buffer|global|flat|scratch)_store_(dwordx[34]|b96|b128)$")


def test_no_valu_write_to_wide_store_data_right_behind_the_store(asm):
    bad = []
    for src, text in asm.items():
        for name, ins, _ in _functions(text):
            for i, (t, _) in enumerate(ins[:-1]):
                op, ops = _operands(t)
                if not WIDE_STORE.match(op):
                    continue
                data = _regs(ops[1] if op.startswith(("global", "flat", "scratch")) else ops[0])
                nxt, _ = ins[i + 1]
                nop, nops = _operands(nxt)
                if nop.startswith("v_") and not nop.startswith(("v_cmp", "v_readfirstlane", "v_readlane")) \
                        and _regs(nops[0]) & data:
                    bad.append(f"{src} {name[:60]}: {t} / {nxt}")
    assert not bad, "\n".join(bad[:10])


def test_inline_asm_lds_reads_untouched_until_their_wait(asm):
    checked, bad = 0, []
    for src, text in asm.items():
        for name, ins, labels in _functions(text):
            def succ(j):
                t = ins[j][0]
                op = t.split()[0]
                if op == "s_branch":
                    return [labels[t.split()[1]]]
                if op.startswith("s_cbranch"):
                    return [labels[t.split()[1]], j + 1]
                if op == "s_endpgm":
                    return []
                return [j + 1]

            for i, (t, in_asm) in enumerate(ins):
                op, ops = _operands(t)
                if not (in_asm and op.startswith("ds_read")):
                    continue
                checked += 1
                dst = _regs(ops[0])
                seen, stack = set(), [i + 1]
                while stack:
                    j = stack.pop()
                    if j in seen or j >= len(ins):
                        continue
                    seen.add(j)
                    tj, aj = ins[j]
                    opj, opsj = _operands(tj)
                    if opj == "s_waitcnt" and "lgkmcnt(0)" in tj:
                        continue
                    if not (aj and opj.startswith("ds_read")):
                        touched = set().union(*[_regs(o) for o in opsj]) if opsj else set()
                        if touched & dst:
                            bad.append(f"{src} {name[:60]}: {t} / {tj}")
                            continue
                    stack.extend(succ(j))
    assert checked > 0, "no inline-asm LDS reads found: the scan no longer matches the sources"
    assert not bad, "\n".join(bad[:10])


def _sregs(tok):
    """SGPRs named by one operand (s7, s[4:7], vcc -> s106/s107 are not modelled: vcc reads are listed as 'vcc')."""
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return {("s", i) for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    m = re.match(r"s(\d+)$", tok)
    if m:
        return {("s", int(m.group(1)))}
    return {("vcc", 0)} if tok in ("vcc", "vcc_lo", "vcc_hi") else set()


def _valu_sgpr_writes(t):
    """SGPRs a VALU instruction writes (lane reads, compares and carry outputs)."""
    op, ops = _operands(t)
    if not op.startswith("v_") or not ops or not ops[0]:
        return set()
    if op.startswith(("v_readlane", "v_readfirstlane")):
        return _sregs(ops[0])
    if op.startswith("v_cmp"):
        return _sregs(ops[0]) if op.endswith("_e64") else {("vcc", 0)}
    if re.match(r"v_(add|sub|subrev)_co|v_div_scale|v_mad_(u|i)64", op):
        return _sregs(ops[1]) if len(ops) > 1 and op.endswith("_e64") else {("vcc", 0)}
    return set()


def _wait_states(t):
    op, ops = _operands(t)
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


VMEM = re.compile(r"^(buffer|global|flat|scratch)_")


def test_vmem_reads_no_sgpr_a_valu_wrote_within_five_wait_states(asm):
    # A VALU write of an SGPR needs 5 wait states before a vector-memory
    # instruction reads that SGPR (resource, offset or address).  The compiler
    # inserts them for its own instructions but not for inline asm, so a
    # spilled SGPR restored by v_readlane right before an inline-asm store
    # makes the store use a stale resource or offset.
    checked, bad = 0, []
    for src, text in asm.items():
        for name, ins, _ in _functions(text):
            for i, (t, _) in enumerate(ins):
                op, ops = _operands(t)
                if not VMEM.match(op):
                    continue
                reads = set().union(*[_sregs(o) for o in ops]) if ops else set()
                if not reads:
                    continue
                checked += 1
                ws, j = 0, i - 1
                while j >= 0 and ws < 5:
                    tj = ins[j][0]
                    if tj.split()[0] in ("s_endpgm",) or tj.startswith("s_cbranch") or tj.startswith("s_branch"):
                        break
                    if _valu_sgpr_writes(tj) & reads:
                        bad.append(f"{src} {name[:60]}: {tj} / {t} ({ws} wait states)")
                        break
                    ws += _wait_states(tj)
                    j -= 1
    assert checked > 0
    assert not bad, "\n".join(bad[:10])


def test_no_valu_write_to_wide_store_data_within_its_window(asm):
    # Every store wider than 8 bytes keeps its data registers free of VALU
    # writes for a window of wait states: 4 behind the inline-asm stores (their
    # trailing s_nop 3), and 2 behind compiler-emitted ones (the compiler's own
    # hazard model for this processor family, which the code it emits follows;
    # a write directly behind a store is what lost data on gfx950).
    bad = []
    for src, text in asm.items():
        for name, ins, _ in _functions(text):
            for i, (t, in_asm) in enumerate(ins):
                op, ops = _operands(t)
                if not WIDE_STORE.match(op):
                    continue
                window = 4 if in_asm else 2
                data = _regs(ops[1] if op.startswith(("global", "flat", "scratch")) else ops[0])
                ws, j = 0, i + 1
                while j < len(ins) and ws < window:
                    nxt = ins[j][0]
                    nop, nops = _operands(nxt)
                    if nop.startswith(("s_cbranch", "s_branch", "s_endpgm")):
                        break
                    if nop.startswith("v_") and not nop.startswith(("v_cmp", "v_readfirstlane", "v_readlane")) \
                            and nops and _regs(nops[0]) & data:
                        bad.append(f"{src} {name[:60]}: {t} / {nxt} ({ws} wait states)")
                        break
                    ws += _wait_states(nxt)
                    j += 1
    assert not bad, "\n".join(bad[:10])
