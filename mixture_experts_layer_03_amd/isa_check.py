"""Wait-state check of the gfx950 assembly around the inline-asm global -> LDS copies.

The compiler inserts the wait states the CDNA instruction set requires between
dependent instructions it generates, but it does not look inside inline asm.  The
copies in csrc/common.h therefore carry their own; this module verifies, on the
device assembly of every source, that each copy (global_load_lds_*) obeys:

  * SGPR base: the base pair must not have been written by a VALU instruction
    (v_readlane_b32, v_readfirstlane_b32, v_cmp*, carry-out adds, ...) within the
    5 preceding wait states - a VMEM instruction may otherwise read the old value
    (this produced wild addresses when the compiler restored a spilled base with
    v_readlane right before a copy);
  * M0: at least 1 wait state after an SALU write of M0.

Each instruction counts as one wait state and s_nop N as N + 1.  Labels end the
backward scan (the check is local to straight-line code, which is where the copies'
operands are produced).
"""
from __future__ import annotations

import re

_COPY = re.compile(r"^global_load_lds_\w+\s+v\[?\d+(?::\d+\])?,\s+(s\[(\d+):(\d+)\]|off)")
_SGPR = re.compile(r"s\[(\d+):(\d+)\]|\bs(\d+)\b")
_VALU_SDST = re.compile(r"^(v_readlane_b32|v_readfirstlane_b32|v_cmp\w*|v_cmpx\w*|v_add_co_u32\w*|v_sub_co_u32\w*"
                        r"|v_subrev_co_u32\w*|v_addc_co_u32\w*|v_subb_co_u32\w*|v_subbrev_co_u32\w*"
                        r"|v_mad_u64_u32\w*|v_mad_i64_i32\w*|v_div_scale\w*)\s+(\S+?),")
_M0_WRITE = re.compile(r"^s_\w+\s+m0\b")


def _sgprs(tok: str) -> set:
    out = set()
    for m in _SGPR.finditer(tok):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _dst(ins: str) -> str:
    parts = ins.split(None, 1)
    return parts[1].split(",")[0].strip() if len(parts) > 1 else ""


def check(asm: str) -> list:
    """Violations (one string each) in the device assembly text of one source."""
    bad = []
    fn = "?"
    hist = []  # straight-line instructions since the last label, newest last
    for raw in asm.splitlines():
        line = raw.split(";", 1)[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            if re.match(r"^_Z\w+:$", line):
                fn = line[:-1]
            hist = []
            continue
        if line.startswith("."):
            continue
        m = _COPY.match(line)
        if m:
            base = _sgprs(m.group(1)) if m.group(1) != "off" else set()
            ws = 0
            m0_seen = False
            for prev in reversed(hist):
                if _M0_WRITE.match(prev) and ws < 1:
                    bad.append(f"{fn}: M0 written {ws} wait states before `{line}`")
                    m0_seen = True
                if base and ws < 5:
                    v = _VALU_SDST.match(prev)
                    if v and _sgprs(_dst(prev)) & base:
                        bad.append(f"{fn}: `{prev}` {ws} wait states before `{line}`")
                        break
                    if prev.startswith("s_") and _sgprs(_dst(prev)) & base and not m0_seen:
                        # the most recent writer of (part of) the base is an SALU op:
                        # only older writes of the other half can still matter
                        base = base - _sgprs(_dst(prev))
                n = re.match(r"^s_nop\s+(\d+)", prev)
                ws += int(n.group(1)) + 1 if n else 1
                if ws >= 5 or (not base and ws >= 1):
                    break
        hist.append(line)
        if len(hist) > 16:
            hist = hist[-16:]
    return bad
