"""Static check of the wait states around inline-asm MFMAs: the bf16 softmax kernel and
the merged dK/dV softmax backward kernel.

Both kernels write their MFMAs as inline asm (to pin register classes), so the compiler's
hazard recognizer does not see them as matrix instructions and inserts no wait states for
them.  The kernels place their own (register-tied s_nop fences), but the compiler is
still free to put a VALU move (a rematerialised constant, a register copy) right before
an MFMA that reads its result.  This module compiles the sources to gfx950 assembly and
checks, on the control-flow graph of each such kernel, the CDNA3/CDNA4 rules that apply
to these instructions:

  - a VALU write of a VGPR or AGPR that an MFMA then reads (A, B or C operand): at least
    2 wait states between them;
  - an MFMA's result read or overwritten by the VALU, or read by a store: NumPasses + 4
    wait states (NumPasses + 3, plus one on gfx950): 12 after the 8-pass 32x32x16 bf16
    MFMA (also taken for the shorter 16x16x32), 20 after the 16-pass 32x32x64 fp8 one
    (the count hipcc's own hazard recognizer inserts after that builtin);
  - an MFMA's C operand overwritten by the VALU: NumPasses + 3 wait states;
  - an M0 write (the LDS destination of a DMA copy) then the copy: 1 wait state;
  - a VALU write of an SGPR (v_readfirstlane, ...) then a vector memory instruction that
    reads it (a copy's base address): 5 wait states.

A wait state is one issued instruction; s_nop N counts N + 1.

It also checks the sources whose kernels copy into LDS with the inline-asm DMA (which
writes M0, a register the compiler reserves and does not protect around inline asm):
no compiler-generated instruction there may use M0.

Used by build() and by a CPU test; the build fails on any violation.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

VALU_TO_MFMA = 2
MFMA_TO_VALU_READ = 12
MFMA_SRCC_TO_VALU_WRITE = 11
VMEM_SGPR_AFTER_VALU = 5
# MFMAs with more passes than the 8 the defaults above are for
PASSES = {"v_mfma_f32_32x32x64_f8f6f4": 16, "v_mfma_scale_f32_32x32x64_f8f6f4": 16}
MAX_PASSES = max(PASSES.values())


def _passes(op: str) -> int:
    return PASSES.get(op, 8)


# (source file under csrc/, mangled-name prefixes of its kernels written with asm MFMAs)
TARGETS = (("softmax_bf16.hip", ("_ZN3vdn17softmax_sw_kernel", "_ZN3vdn22softmax_sw_redo_kernel",
                                 "_ZN3vdn18softmax_sw8_kernel", "_ZN3vdn23softmax_sw8_redo_kernel")),
           ("backward.hip", ("_ZN3vdn21softmax_bwd_kv_kernel",)))
PREFIXES = tuple(p for _, ps in TARGETS for p in ps)
# sources whose kernels write M0 in inline asm (the LDS DMA copies)
M0_SOURCES = ("softmax_bf16.hip", "backward.hip", "delta_bf16.hip", "mxfp8.hip", "proj_gemm.hip", "linear_bf16.hip")

_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")
_STORE = ("ds_write", "ds_store", "global_store", "buffer_store", "scratch_store", "flat_store")
_LOAD = ("ds_read", "ds_load", "global_load", "buffer_load", "scratch_load", "flat_load")


def _regs(text: str) -> set[tuple[str, int]]:
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


class _Inst:
    __slots__ = ("op", "dst", "src", "srcc", "nop", "text")

    def __init__(self, op, dst, src, srcc, nop, text):
        self.op, self.dst, self.src, self.srcc, self.nop, self.text = op, dst, src, srcc, nop, text

    @property
    def valu(self) -> bool:
        return self.op.startswith("v_") and not self.op.startswith("v_mfma")

    @property
    def mfma(self) -> bool:
        return self.op.startswith("v_mfma")


def _parse(line: str):
    line = line.split(";")[0].strip()
    if not line:
        return None
    parts = line.split(None, 1)
    op, rest = parts[0], (parts[1] if len(parts) > 1 else "")
    operands = [x.strip() for x in re.split(r",(?![^\[]*\])", rest)] if rest else []
    if op == "s_nop":
        return _Inst(op, set(), set(), set(), int(operands[0], 0) + 1, line)
    if op.startswith("s_") or op.startswith("v_cmp"):
        # scalar instructions touch no vector registers; v_cmp writes VCC or SGPRs
        src = set()
        for x in (operands[1:] if op.startswith("v_cmp") else []):
            src |= _regs(x)
        return _Inst(op, set(), src, set(), 1, line)
    if op.startswith(_STORE):
        src = set()
        for x in operands:
            src |= _regs(x)
        return _Inst(op, set(), src, set(), 1, line)
    dst = _regs(operands[0]) if operands else set()
    src = set()
    for x in operands[1:]:
        src |= _regs(x)
    srcc = _regs(operands[3]) if op.startswith("v_mfma") and len(operands) > 3 else set()
    return _Inst(op, dst, src, srcc, 1, line)


def _kernels(asm: str, prefixes=PREFIXES) -> dict[str, list]:
    """Kernel name -> list of (label or None, instruction or None) in program order."""
    out, cur, name = {}, None, None
    for raw in asm.split("\n"):
        if re.match(r"^[A-Za-z_][\w.]*:", raw) and not raw.startswith("."):
            label = raw.split(":")[0]
            if label.startswith(tuple(prefixes)):
                name, cur = label, []
                out[name] = cur
                continue
        if cur is None:
            continue
        if raw.startswith("\ts_endpgm") or raw.strip() == "s_endpgm":
            cur.append((None, _parse("s_endpgm")))
            cur = None
            continue
        m = re.match(r"^(\.LBB\d+_\d+):", raw)
        if m:
            cur.append((m.group(1), None))
            continue
        if raw.startswith("\t") and not raw.startswith("\t."):
            inst = _parse(raw)
            if inst is not None:
                cur.append((None, inst))
    return out


_BIG = 99  # exec depth after an exec write of unknown effect


def _exec_effect(inst, d: int) -> int:
    """Divergence depth after `inst` (0: all lanes of the wave active)."""
    if inst is None:
        return d
    if inst.op.startswith("s_") and "saveexec" in inst.op:
        return min(d + 1, _BIG)  # entry of a divergent region
    parts = inst.text.split(None, 1)
    ops = [x.strip() for x in parts[1].split(",")] if len(parts) > 1 else []
    if ops and ops[0] == "exec":
        if inst.op == "s_or_b64" and len(ops) > 1 and ops[1] == "exec":
            return max(d - 1, 0)  # end of a divergent region: the saved mask comes back
        if inst.op == "s_xor_b64" and d > 0:
            return d  # the else part of a divergent region
        return _BIG
    return d


def _preds(items):
    """Index -> list of predecessor instruction indices (program order plus branches).

    The kernels are launched with whole waves (workgroups of a multiple of 64 threads), so
    every lane is active at entry.  A forward pass tracks the divergence depth (saveexec
    regions the compiler opens, their s_or_b64 exec restores); an s_cbranch_execz where
    the depth is 0 cannot be taken (exec is all ones), and its jump is not an edge.  The
    compiler emits such branches around uniform code too."""
    idx_of_label = {}
    for i, (lab, _) in enumerate(items):
        if lab:
            idx_of_label[lab] = i
    n = len(items)
    succ = {i: [] for i in range(n)}
    for i, (lab, inst) in enumerate(items):
        if i + 1 < n:
            uncond = inst is not None and (inst.op in ("s_branch", "s_endpgm", "s_setpc_b64"))
            if not uncond:
                succ[i].append((i + 1, False))
        if inst is not None and inst.op.startswith(("s_branch", "s_cbranch")):
            target = inst.text.split()[-1]
            if target in idx_of_label:
                succ[i].append((idx_of_label[target], inst.op == "s_cbranch_execz"))
    depth_in = [None] * n
    if n:
        depth_in[0] = 0
    work = [0] if n else []
    while work:
        i = work.pop()
        out = _exec_effect(items[i][1], depth_in[i])
        for j, _ in succ[i]:
            if depth_in[j] is None or out > depth_in[j]:
                depth_in[j] = out
                work.append(j)
    preds = {i: [] for i in range(n)}
    for i in range(n):
        if depth_in[i] is None:
            continue  # unreachable
        out = _exec_effect(items[i][1], depth_in[i])
        for j, execz in succ[i]:
            if execz and out == 0:
                continue
            preds[j].append(i)
    return preds


def _search(items, preds, start, need, hit):
    """Walk back from instruction `start` through the CFG while fewer than `need` wait
    states separate it; return the first instruction for which hit(inst) holds.  `need`
    is a number or a function of the instruction found (then the walk goes back as far
    as the largest requirement and reports a hit only inside its own)."""
    need_of = need if callable(need) else (lambda inst: need)
    reach = need if not callable(need) else MAX_PASSES + 4
    stack = [(p, 0) for p in preds[start]]
    seen = set()
    while stack:
        i, waited = stack.pop()
        if (i, waited) in seen:
            continue
        seen.add((i, waited))
        lab, inst = items[i]
        if inst is None:
            stack.extend((p, waited) for p in preds[i])
            continue
        if hit(inst) and waited < need_of(inst):
            return inst, waited
        waited += inst.nop
        if waited < reach:
            stack.extend((p, waited) for p in preds[i])
    return None


_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


def _sregs(text: str) -> set[int]:
    out = set()
    for m in _SREG.finditer(text):
        if m.group(1):
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _valu_sgpr_dst(inst) -> set[int]:
    """SGPRs a VALU instruction writes (v_readfirstlane, v_readlane, a v_cmp into SGPRs)."""
    if not inst.valu:
        return set()
    ops = inst.text.split(None, 1)
    return _sregs(ops[1].split(",")[0]) if len(ops) > 1 else set()


def _writes_m0(inst) -> bool:
    ops = inst.text.split(None, 1)
    return inst.op.startswith("s_") and len(ops) > 1 and ops[1].split(",")[0].strip() == "m0"


def check_asm(asm: str, prefixes=PREFIXES) -> list[str]:
    problems = []
    kernels = _kernels(asm, prefixes)
    if not kernels:
        return ["none of the kernels " + ", ".join(prefixes) + " in the assembly"]
    for name, items in kernels.items():
        preds = _preds(items)
        for i, (lab, inst) in enumerate(items):
            if inst is None:
                continue
            if inst.op.startswith(("global_", "buffer_")):
                # a vector memory instruction reading an SGPR the VALU wrote: 5 wait states
                # (the compiler places them for its own memory instructions, not for asm)
                sr = _sregs(inst.text.split(None, 1)[1]) if " " in inst.text else set()
                r = _search(items, preds, i, VMEM_SGPR_AFTER_VALU, lambda p: bool(_valu_sgpr_dst(p) & sr))
                if r:
                    problems.append(f"{name}: VALU write of an SGPR '{r[0].text}' then memory read of it after {r[1]} wait states: '{inst.text}'")
            if inst.op.startswith("global_load_lds") or (inst.op.startswith("buffer_load") and " lds" in inst.text):
                r = _search(items, preds, i, 1, _writes_m0)
                if r:
                    problems.append(f"{name}: M0 write '{r[0].text}' then LDS DMA after {r[1]} wait states: '{inst.text}'")
            if inst.mfma:
                reads = inst.src
                r = _search(items, preds, i, VALU_TO_MFMA, lambda p: p.valu and (p.dst & reads))
                if r:
                    problems.append(f"{name}: VALU write '{r[0].text}' then MFMA read after {r[1]} wait states: '{inst.text}'")
            if inst.valu or inst.op.startswith(_STORE):
                touched = inst.src | (inst.dst if inst.valu else set())
                r = _search(items, preds, i, lambda p: max(MFMA_TO_VALU_READ, _passes(p.op) + 4),
                            lambda p: p.mfma and (p.dst & touched))
                if r:
                    problems.append(f"{name}: MFMA result '{r[0].text}' used after {r[1]} wait states: '{inst.text}'")
                if inst.valu and inst.dst:
                    w = inst.dst
                    r = _search(items, preds, i, lambda p: max(MFMA_SRCC_TO_VALU_WRITE, _passes(p.op) + 3),
                                lambda p: p.mfma and (p.srcc & w) and not (p.dst & w))
                    if r:
                        problems.append(f"{name}: MFMA C operand '{r[0].text}' overwritten after {r[1]} wait states: '{inst.text}'")
    return problems


def check_m0(asm: str) -> list[str]:
    """Compiler-generated instructions (outside inline-asm blocks) that name M0."""
    problems, in_asm = [], False
    for raw in asm.split("\n"):
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
        elif t.startswith(";;#ASMEND"):
            in_asm = False
        elif not in_asm and t and not t.startswith((".", ";")) and re.search(r"\bm0\b", t.split(";")[0]):
            problems.append(f"compiler-generated use of M0 beside the inline-asm LDS copies: '{t}'")
    return problems


def kernel_asm(src: str) -> str:
    """gfx950 assembly of a source file, compiled with the library's flags."""
    from .build import FLAGS, HIPCC
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "kernels.s")
        flags = [f for f in FLAGS if f != "-fPIC"]
        r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} to assembly failed:\n" + r.stderr[-4000:])
        with open(out) as fh:
            return fh.read()


def check(src: str | None = None) -> list[str]:
    """Problems found in one source file (every checked kernel in it), or, with no
    argument, in each of the library's sources that holds asm-MFMA kernels."""
    if src is not None:
        return check_asm(kernel_asm(src))
    from .build import CSRC
    problems = []
    asm = {}
    for name, prefixes in TARGETS:
        asm[name] = kernel_asm(os.path.join(CSRC, name))
        problems += check_asm(asm[name], prefixes)
    for name in M0_SOURCES:
        problems += [f"{name}: {p}" for p in check_m0(asm.get(name) or kernel_asm(os.path.join(CSRC, name)))]
    return problems


if __name__ == "__main__":
    import sys
    found = check(sys.argv[1] if len(sys.argv) > 1 else None)
    print("\n".join(found) if found else "no MFMA wait-state violations, no compiler use of M0 beside the LDS copies")
    sys.exit(1 if found else 0)
