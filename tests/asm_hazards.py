"""Wait-state check of compiled gfx950 kernels (test helper, no GPU).

The decode kernels issue their matrix instructions as inline asm, so the
compiler does not insert the wait states the hardware needs around them.  The
kernels add them where they are due (pins, s_nop guards, drains); this scan
checks the compiled code instead of trusting that:

* an MFMA may read a register written by a vector (VALU) instruction only
  after at least ``VALU_TO_MFMA`` wait states (2 on gfx950, the padding the
  compiler itself emits for its own MFMAs);
* an instruction other than an MFMA may read or write a register an MFMA
  wrote only after the wait states ``mfma_to_other`` gives for that MFMA (the
  padding the compiler emits after its own: 12 after the FP8 16x16x128, 8
  after the bf16 16x16x32).

Wait states between two instructions: one per instruction in between, N + 1
per ``s_nop N``.  The scan follows the control flow: at a branch target the
state is the worst case over the fall-through and every branch to it, and the
function is scanned twice so that loop back edges are seen.
"""
from __future__ import annotations

import re

VALU_TO_MFMA = 2
_CAP = 64  # distances beyond every rule


def mfma_to_other(op: str) -> int:
    return 12 if "f8f6f4" in op else 8


def _regs(tok: str) -> set:
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", tok):
        if m.group(1):
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((m.group(1), r))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _parse(body: str):
    """[(kind, payload)]: ("label", name) or ("ins", (op, operands, text))."""
    items = []
    for line in body.split("\n"):
        t = line.split(";")[0].strip()
        if not t or t.startswith("."):
            m = re.match(r"^(\.LBB\w+):", line.strip())
            if m:
                items.append(("label", m.group(1)))
            continue
        if t.endswith(":"):
            items.append(("label", t[:-1]))
            continue
        op = t.split()[0]
        rest = t[len(op):].strip()
        parts = [p.strip() for p in re.split(r",(?![^\[]*\])", rest)] if rest else []
        items.append(("ins", (op, parts, t)))
    return items


def _merge(a: dict, b: dict) -> dict:
    out = dict(a)
    for k, v in b.items():
        out[k] = min(out.get(k, _CAP), v)
    return out


def _advance(state: dict, n: int) -> dict:
    return {k: v + n for k, v in state.items() if v + n < _CAP}


def check(body: str) -> list[str]:
    """Violations in one kernel's asm text (empty list: none)."""
    items = _parse(body)
    at_label: dict[str, tuple[dict, dict]] = {}
    found: dict[str, str] = {}
    for _ in range(2):
        valu: dict = {}   # register -> wait states since a VALU write
        mfma: dict = {}   # register -> wait states since an MFMA write
        need: dict = {}   # register -> wait states its MFMA requires
        reachable = True
        for kind, payload in items:
            if kind == "label":
                v2, m2 = at_label.get(payload, ({}, {}))
                if reachable:
                    valu, mfma = _merge(valu, v2), _merge(mfma, m2)
                else:
                    valu, mfma = dict(v2), dict(m2)
                reachable = True
                continue
            op, parts, text = payload
            if not reachable:
                continue
            n = int(parts[0], 0) + 1 if op == "s_nop" and parts else 1
            if op.startswith("v_mfma"):
                srcs = set().union(*[_regs(p) for p in parts[1:]]) if len(parts) > 1 else set()
                for r in sorted(srcs):
                    if valu.get(r, _CAP) < VALU_TO_MFMA:
                        found.setdefault(text, f"VALU write {valu[r]} wait states before: {text}")
                valu, mfma = _advance(valu, n), _advance(mfma, n)
                for r in _regs(parts[0]) if parts else ():
                    mfma[r] = 0
                    need[r] = max(need.get(r, 0), mfma_to_other(op))  # the stricter, across paths
                    valu.pop(r, None)
                continue
            if op != "s_nop":
                touched = set().union(*[_regs(p) for p in parts]) if parts else set()
                for r in sorted(touched):
                    if mfma.get(r, _CAP) < need.get(r, 12):
                        found.setdefault(text, f"MFMA result {mfma[r]} wait states before: {text}")
            valu, mfma = _advance(valu, n), _advance(mfma, n)
            if op.startswith("v_") and parts:
                for r in _regs(parts[0]):
                    valu[r] = 0
                    mfma.pop(r, None)
            if op.startswith("s_cbranch") or op == "s_branch":
                tgt = parts[0] if parts else ""
                v2, m2 = at_label.get(tgt, ({}, {}))
                at_label[tgt] = (_merge(v2, valu), _merge(m2, mfma))
            if op in ("s_branch", "s_endpgm", "s_setpc_b64"):
                reachable = False
    return sorted(found.values())


def kernels(asm: str, pattern: str) -> dict[str, str]:
    """Kernel name -> body (up to s_endpgm) for the kernels whose mangled
    name matches ``pattern``."""
    out = {}
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        name = m.group(1)
        if not re.search(pattern, name):
            continue
        end = asm.find("s_endpgm", m.end())
        out[name] = asm[m.end():end]
    return out
