"""Checks on the device assembly of inline-asm MFMAs (test infrastructure).

The bf16 prefill kernel issues the MFMAs of its S block as inline asm, so that
their accumulators stay in VGPRs.  The compiler inserts no hazard wait states
around inline asm and may reuse or copy registers right after an asm
statement, so two rules are checked on the compiled code:

* operands (write after read): once an asm MFMA has issued, no instruction may
  write its A or B registers before another MFMA has issued or WAR_WAIT wait
  states (s_nop) have passed;
* accumulator (read after write): no instruction other than an MFMA continuing
  the chain may read an asm MFMA's accumulator before RAW_WAIT wait states.

The asm blocks themselves end their chains with 20 wait states.  Only wait
states inside asm blocks count (those outside may sit on a path that a branch
skips), and the scan restarts after an unconditional branch; a conditional
branch keeps the state, so a skipped block is checked as if it ran.
"""
from __future__ import annotations

import re

WAR_WAIT = 16
RAW_WAIT = 18

_WRITERS = ("v_", "ds_read", "global_load", "buffer_load", "scratch_load", "flat_load")


def _regs(tok: str) -> set[int]:
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def functions(asm: str) -> dict[str, list[str]]:
    """Kernel name -> its instruction lines (from the label to s_endpgm)."""
    out, name, body = {}, None, []
    for ln in asm.split("\n"):
        m = re.match(r"^([A-Za-z_][\w.$]*):\s*(;.*)?$", ln)
        if m and not ln.startswith(".") and name is None:
            name, body = m.group(1), []
            continue
        if name is not None:
            body.append(ln)
            if ln.strip().startswith("s_endpgm"):
                out[name] = body
                name = None
    return out


def violations(lines: list[str]) -> list[str]:
    """Both rules over one function's lines; returns a description per violation."""
    bad = []
    in_asm = False
    war = None          # (line, operand regs, waited)
    raw = []            # [line, accumulator regs, waited]
    for i, ln in enumerate(lines):
        t = ln.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        parts = t.replace(",", " ").split()
        op = parts[0]
        if op in ("s_branch", "s_setpc_b64", "s_endpgm"):
            # nothing falls through: the next line starts another path
            war, raw = None, []
            continue
        if op == "s_nop" and in_asm:   # only the asm blocks' own wait states count
            n = int(parts[1], 0) + 1
            if war is not None:
                war = (war[0], war[1], war[2] + n)
                if war[2] >= WAR_WAIT:
                    war = None
            for r in raw:
                r[2] += n
            raw = [r for r in raw if r[2] < RAW_WAIT]
            continue
        if op.startswith("v_mfma"):
            dst = _regs(parts[1])
            if in_asm:
                war = (i, _regs(parts[2]) | _regs(parts[3]), 0)
                raw = [r for r in raw if not (r[1] & dst)]
                raw.append([i, dst, 0])
            else:
                war = None
            continue
        if op.startswith("s_"):
            continue
        # registers written (first operand of VALU and loads) and read
        writes = set()
        if op.startswith(_WRITERS) and len(parts) > 1 and not (op.startswith("buffer_load") and parts[-1] == "lds"):
            writes = _regs(parts[1])
        srcs = parts[1:] if ("store" in op or op.startswith("ds_write")) else parts[2:]
        reads = set()
        for s in srcs:
            reads |= _regs(s)
        if war is not None and writes & war[1]:
            bad.append(f"{t!r} overwrites an operand of the asm MFMA {lines[war[0]].strip()!r}")
        for r in raw:
            if reads & r[1]:
                bad.append(f"{t!r} reads the accumulator of the asm MFMA {lines[r[0]].strip()!r} "
                           f"after {r[2]} wait states")
    return bad
