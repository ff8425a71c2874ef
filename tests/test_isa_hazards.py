"""Wait states around the inline-assembly MFMAs, checked on the built code.

The MLA decode issues its score MFMAs from inline assembly (their results go
to VGPRs), so the compiler's hazard recognizer does not see them as MFMAs.
The code relies on two gfx950 rules, and this test checks both on the
assembly that hipcc produces for every kernel of the file, with the
library's own flags (CPU only: hipcc cross-compiles for gfx950):

* a VALU write of a VGPR must be at least 2 wait states ahead of an MFMA
  that reads it (the operands here come from LDS reads and global loads,
  which the memory counters cover instead);
* after an MFMA, no VALU, LDS or memory instruction may read or overwrite
  its result for the MFMA's passes plus a few wait states; the test asks
  for 12 (an 8-pass MFMA plus 4), the asm provides 19.  An MFMA that
  accumulates onto exactly the same registers may follow at once.

One wait state per instruction, N + 1 per ``s_nop N``; the windows follow
every control-flow path (into a label from each branch to it and from the
instruction above it, out of a conditional branch both ways).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_38_amd import build as B

VALU_TO_MFMA = 2
MFMA_TO_USE = 12

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")


def _regs(operand: str) -> set[tuple[str, int]]:
    out = set()
    for m in _REG.finditer(operand):
        kind = m.group(1)
        lo, hi = (int(m.group(2)), int(m.group(3))) if m.group(2) else (int(m.group(4)), int(m.group(4)))
        out.update((kind, r) for r in range(lo, hi + 1))
    return out


def _parse(line: str):
    code = line.split(";", 1)[0].strip()
    if not code:
        return None
    if re.match(r"^[.\w]+:$", code):
        return ("label", code, [])
    if code.startswith("."):
        return None
    parts = code.split(None, 1)
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return ("insn", parts[0], ops)


def _wait_states(op: str, ops: list[str]) -> int:
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def _target(ops: list[str]) -> str | None:
    return ops[0] if ops else None


def _flow(body):
    """Label positions, and for each label the branches that jump to it."""
    where = {op[:-1]: i for i, (k, op, _) in enumerate(body) if k == "label"}
    into: dict[str, list[int]] = {}
    for i, (k, op, ops) in enumerate(body):
        if k == "insn" and (op == "s_branch" or op.startswith("s_cbranch")) and _target(ops) in where:
            into.setdefault(_target(ops), []).append(i)
    return where, into


def _before(body, flow, j: int, need: int, visit) -> None:
    """Call visit(insn) for every instruction that can run within `need`
    wait states before position j + 1, along every control-flow path."""
    where, into = flow
    while need > 0 and j >= 0:
        k, op, ops = body[j]
        if k == "label":
            for b in into.get(op[:-1], []):
                _before(body, flow, b, need, visit)
            prev = body[j - 1] if j > 0 else None
            if prev is None or prev[1] in ("s_branch", "s_setpc_b64", "s_endpgm"):
                return
            j -= 1
            continue
        visit(k, op, ops)
        need -= _wait_states(op, ops)
        j -= 1


def _after(body, flow, j: int, need: int, visit) -> None:
    """Call visit(insn) for every instruction that can run within `need`
    wait states after position j - 1, along every control-flow path."""
    where, _ = flow
    while need > 0 and j < len(body):
        k, op, ops = body[j]
        if k == "label":
            j += 1
            continue
        visit(k, op, ops)
        need -= _wait_states(op, ops)
        if op == "s_endpgm":
            return
        if op == "s_branch":
            j = where[_target(ops)]
            continue
        if op.startswith("s_cbranch"):
            _after(body, flow, where[_target(ops)], need, visit)
        j += 1


def _kernels(asm: str):
    lines = asm.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\w+:", l)]
    for s in starts:
        e = next(i for i in range(s + 1, len(lines)) if lines[i].startswith(".Lfunc_end"))
        body = [p for p in (_parse(l) for l in lines[s + 1:e]) if p is not None]
        yield lines[s].split(":")[0], body


def _check(body) -> list[str]:
    errs = []
    flow = _flow(body)
    for i, (kind, op, ops) in enumerate(body):
        if kind != "insn" or not op.startswith("v_mfma") or not ops[0].startswith("v"):
            continue
        me = f"{op} {','.join(ops)}"
        dst = _regs(ops[0])
        srcs = set().union(*(_regs(o) for o in ops[1:]))

        def early_write(k2, op2, ops2):
            if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2 and _regs(ops2[0]) & srcs:
                errs.append(f"{me}: operand written by '{op2} {','.join(ops2)}' too close")

        def early_use(k2, op2, ops2):
            touched = set().union(*(_regs(o) for o in ops2)) if ops2 else set()
            if touched & dst:
                chain = op2.startswith("v_mfma") and _regs(ops2[0]) == dst and _regs(ops2[-1]) == dst and \
                    not (set().union(*(_regs(o) for o in ops2[1:-1])) & dst)
                if not chain:
                    errs.append(f"{me}: result used by '{op2} {','.join(ops2)}' too early")

        _before(body, flow, i - 1, VALU_TO_MFMA, early_write)
        _after(body, flow, i + 1, MFMA_TO_USE, early_use)
    return errs


def test_inline_mfma_wait_states(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = os.path.join(B.CSRC, "pkv_mla.hip")
    out = tmp_path / "mla.s"
    cmd = [hipcc, *B.HIPCC_FLAGS, f"-I{B.INCLUDE}", "--offload-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    n_asm_mfma, errs = 0, []
    for name, body in _kernels(asm):
        n_asm_mfma += sum(1 for k, op, ops in body if k == "insn" and op.startswith("v_mfma") and ops[0].startswith("v"))
        errs += [f"{name[:60]}: {e}" for e in _check(body)]
    assert n_asm_mfma > 0, "no VGPR-result MFMAs found: the check would be vacuous"
    assert not errs, "\n".join(errs[:20])


def test_checker_catches_planted_hazards():
    """The checker itself: a VALU write right before an MFMA operand read, and
    a VALU read of an MFMA result right after it, are both reported; a chained
    accumulation and a padded read are not."""
    bad = [
        ("insn", "v_mov_b32_e32", ["v4", "v9"]),
        ("insn", "v_mfma_f32_16x16x32_bf16", ["v[0:3]", "v[4:7]", "v[8:11]", "v[0:3]"]),
        ("insn", "v_add_f32_e32", ["v20", "v1", "v2"]),
    ]
    errs = _check(bad)
    assert any("too close" in e for e in errs) and any("too early" in e for e in errs)
    good = [
        ("insn", "s_nop", ["1"]),
        ("insn", "v_mfma_f32_16x16x32_bf16", ["v[0:3]", "v[4:7]", "v[8:11]", "v[0:3]"]),
        ("insn", "v_mfma_f32_16x16x32_bf16", ["v[0:3]", "v[12:15]", "v[8:11]", "v[0:3]"]),
        ("insn", "s_nop", ["7"]),
        ("insn", "s_nop", ["7"]),
        ("insn", "v_add_f32_e32", ["v20", "v1", "v2"]),
    ]
    # the second MFMA's own window: 16 wait states of nops before the add
    assert _check(good) == []


def test_checker_follows_branches():
    """A VALU write in a block that branches to the MFMA's label is found."""
    body = [
        ("insn", "v_mov_b32_e32", ["v4", "v9"]),
        ("insn", "s_branch", [".LBB0_2"]),
        ("insn", "v_add_f32_e32", ["v30", "v31", "v32"]),
        ("label", ".LBB0_2:", []),
        ("insn", "v_mfma_f32_16x16x32_bf16", ["v[0:3]", "v[4:7]", "v[8:11]", "0"]),
        ("insn", "s_cbranch_scc1", [".LBB0_3"]),
        ("insn", "s_nop", ["7"]),
        ("insn", "s_nop", ["7"]),
        ("label", ".LBB0_3:", []),
        ("insn", "v_add_f32_e32", ["v20", "v1", "v2"]),
    ]
    errs = _check(body)
    assert any("too close" in e and "v_mov_b32_e32" in e for e in errs)
    assert any("too early" in e for e in errs)  # the taken branch skips the nops
