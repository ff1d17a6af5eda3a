"""Static check of the gfx950 assembly that hipcc generates for the kernels.

    python -m moe_grouped_precision_amd.asmcheck <file.s>

The GEMM kernels issue their K-loop vector-memory operations as inline asm
and wait for them with explicit ``s_waitcnt vmcnt``; the compiler does not
see those loads.  This check proves, over the control-flow graph of every
kernel, two properties the compiler can no longer guarantee by itself:

* no instruction reads or overwrites a VGPR that a still-pending vector-memory
  load may write (loads complete in issue order, so after ``vmcnt(N)`` only
  the N newest operations can be pending);
* every vector-memory instruction that takes a scalar (SGPR) address operand
  is at least 5 wait states after the last VALU write of that SGPR.

The dataflow is conservative: at a merge point a register is pending if it
may be pending on any incoming path.  Long branches (s_getpc_b64 / add /
s_setpc_b64, which the compiler emits when a kernel outgrows the short branch
range) are followed to their targets, and a kernel with any block the parsed
control-flow graph does not reach is itself a finding, so the check cannot
silently skip code.  Exit status 1 lists each finding.
"""

from __future__ import annotations

import re
import sys

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_SPAIR = re.compile(r"\bs\[(\d+):(\d+)\]")
_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")
_BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\S+)")
_MAXQ = 64


def _vregs(text):
    out = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _sregs(text):
    out = set()
    for m in _SREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _parse(lines):
    """Split into kernels -> basic blocks of (line_no, instruction)."""
    kernels = []
    cur = None
    for no, raw in enumerate(lines, 1):
        text = raw.split(";")[0].strip()
        if not text:
            continue
        if text.endswith(":"):
            label = text[:-1]
            if not label.startswith("."):
                cur = {"name": label, "blocks": [], "labels": {}}
                kernels.append(cur)
                cur["blocks"].append({"label": label, "ins": []})
                cur["labels"][label] = 0
                continue
            if cur is None:
                continue
            cur["blocks"].append({"label": label, "ins": []})
            cur["labels"][label] = len(cur["blocks"]) - 1
            continue
        if cur is None or text.startswith("."):
            continue
        blk = cur["blocks"][-1]
        blk["ins"].append((no, text))
        op = text.split()[0]
        if op.startswith("s_branch") or op.startswith("s_cbranch") or op == "s_endpgm" or op.startswith("s_setpc"):
            cur["blocks"].append({"label": None, "ins": []})
    return kernels


_LONG_TARGET = re.compile(r"\((\.L\w+)-\.Lpost_getpc\w*\)")


def _successors(kern, bi):
    blk = kern["blocks"][bi]
    succ = []
    last = blk["ins"][-1][1] if blk["ins"] else ""
    op = last.split()[0] if last else ""
    m = _BRANCH.match(last)
    if m and m.group(2) in kern["labels"]:
        succ.append(kern["labels"][m.group(2)])
    if op.startswith("s_setpc"):
        # a long branch: s_getpc_b64, then the target's distance added to the
        # pc in the same block, then s_setpc_b64 -- its target is a successor
        for _, text in blk["ins"]:
            t = _LONG_TARGET.search(text)
            if t and t.group(1) in kern["labels"]:
                succ.append(kern["labels"][t.group(1)])
                break
        else:
            raise ValueError(f"s_setpc_b64 with no recognisable target in block {blk['label']}")
    if op not in ("s_branch", "s_endpgm") and not op.startswith("s_setpc"):
        if bi + 1 < len(kern["blocks"]):
            succ.append(bi + 1)
    return succ


def _merge(a, b):
    if a is None:
        return [set(x) for x in b]
    n = max(len(a), len(b))
    out = []
    for i in range(n):
        s = set()
        if i < len(a):
            s |= a[i]
        if i < len(b):
            s |= b[i]
        out.append(s)
    return out


def _is_vmem(op):
    return op.startswith(("global_", "buffer_", "scratch_", "flat_"))


def _check_kernel(kern, findings):
    nb = len(kern["blocks"])
    state_in = [None] * nb
    state_in[0] = []
    work = [0]
    reported = set()
    # wait states since the last VALU write of each SGPR, per block entry: keep simple,
    # reset at block entry (conservative: treated as just written)
    while work:
        bi = work.pop()
        q = [set(x) for x in state_in[bi]]
        last_valu_sgpr = {}
        count = 0
        for no, text in kern["blocks"][bi]["ins"]:
            op = text.split()[0]
            rest = text[len(op):]
            count += 1
            if op == "s_nop":
                m = re.match(r"\s*(\d+)", rest)
                count += int(m.group(1)) if m else 0
            if op.startswith("s_waitcnt"):
                m = re.search(r"vmcnt\((\d+)\)", text)
                if m:
                    q = q[: int(m.group(1))]
                continue
            if op == "s_endpgm":
                q = []
                continue
            ops = [x.strip() for x in rest.split(",")] if rest.strip() else []
            pend = set().union(*q) if q else set()
            if _is_vmem(op):
                loads_reg = ("load" in op) and ("_lds" not in op) and not re.search(r"\blds\b", rest)
                dst = _vregs(ops[0]) if (loads_reg and ops) else set()
                srcs = set().union(*[_vregs(x) for x in (ops[1:] if loads_reg else ops)]) if ops else set()
                bad = srcs & pend
                if bad and (no, "r") not in reported:
                    reported.add((no, "r"))
                    findings.append(f"line {no}: {text}: reads VGPR v{min(bad)} with a load pending")
                m = _SPAIR.search(rest)
                if m:
                    for r in range(int(m.group(1)), int(m.group(2)) + 1):
                        if r in last_valu_sgpr and count - last_valu_sgpr[r] <= 5 and (no, "s") not in reported:
                            reported.add((no, "s"))
                            findings.append(f"line {no}: {text}: SGPR s{r} written by VALU "
                                            f"{count - last_valu_sgpr[r] - 1} wait states before")
                q.insert(0, dst)
                q = q[:_MAXQ]
                continue
            if op.startswith("v_") or op.startswith("ds_"):
                if op.startswith(("ds_write", "ds_store")):
                    dst, srcs = set(), set().union(*[_vregs(x) for x in ops]) if ops else set()
                else:
                    dst = _vregs(ops[0]) if ops else set()
                    srcs = set().union(*[_vregs(x) for x in ops[1:]]) if len(ops) > 1 else set()
                bad = srcs & pend
                if bad and (no, "r") not in reported:
                    reported.add((no, "r"))
                    findings.append(f"line {no}: {text}: reads VGPR v{min(bad)} with a load pending")
                bad = dst & pend
                if bad and (no, "w") not in reported:
                    reported.add((no, "w"))
                    findings.append(f"line {no}: {text}: overwrites VGPR v{min(bad)} with a load pending")
                if op.startswith("v_") and ops:
                    for r in _sregs(ops[0]):
                        last_valu_sgpr[r] = count
        for s in _successors(kern, bi):
            new = _merge(state_in[s], q)
            if state_in[s] is None or any(i >= len(state_in[s]) or new[i] != state_in[s][i] for i in range(len(new))):
                state_in[s] = new
                work.append(s)


def _unreached(kern):
    """Blocks with instructions that the CFG does not reach from the entry
    (the check would say nothing about them)."""
    seen, stack = {0}, [0]
    while stack:
        b = stack.pop()
        for s in _successors(kern, b):
            if s not in seen:
                seen.add(s)
                stack.append(s)
    return [b for b in range(len(kern["blocks"])) if b not in seen and kern["blocks"][b]["ins"]]


def check(path: str):
    lines = open(path).read().split("\n")
    findings = []
    for kern in _parse(lines):
        if kern["name"].startswith(("amdhsa.", "__hip_cuid")):
            continue   # metadata sections after the kernels
        un = _unreached(kern)
        if un:
            b = kern["blocks"][un[0]]
            findings.append(f"{kern['name']}: {len(un)} block(s) unreachable in the parsed CFG, first at line "
                            f"{b['ins'][0][0]} -- the check would not cover them")
        _check_kernel(kern, findings)
    return findings


if __name__ == "__main__":
    found = check(sys.argv[1])
    for f in found[:50]:
        print(f)
    print(f"{len(found)} finding(s)")
    sys.exit(1 if found else 0)
