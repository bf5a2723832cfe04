"""Static check of gfx950 assembly for the VMEM-after-VALU-SGPR-write hazard
around hand-written memory instructions.

CDNA3/CDNA4 require 5 wait states between a VALU instruction that writes an
SGPR (v_readlane, v_readfirstlane, a VOP3 compare or carry-out, ...) and a
vector-memory instruction that reads that SGPR (for example as the scalar
base address of a global load), and 1 wait state between a scalar write of
M0 and an LDS-DMA load that reads it.  The compiler inserts these for the
instructions it emits itself but not around inline assembly, so a
hand-written ``global_load_lds_dwordx4 v, s[a:b]`` whose base the register
allocator restores with ``v_readlane`` right before it (for instance after a
spill of SGPRs to VGPR lanes) would read a stale base.

Likewise the result of an MFMA written in inline assembly into VGPRs is
taken by the compiler as ready when the statement ends: an instruction that
reads or copies those VGPRs within the MFMA's latency (about a dozen wait
states for the 8-pass 32x32x16 MFMA; 11 are required here) reads stale values,
unless it is the next MFMA of the same accumulation chain (source-C
forwarding).

``scan(asm_text)`` walks every inline-assembly block that holds a global or
buffer load with a scalar base or an LDS destination and counts the wait
states back to the nearest instruction that writes the SGPRs it reads (or
M0), within the basic block; and every inline-assembly MFMA with a VGPR
destination, counting the wait states forward to the first instruction that
touches the destination.  ``hipcc -S`` output of the kernels is the input.
"""
from __future__ import annotations

import re

_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")
_VMEM = re.compile(r"^\s*(global_load|buffer_load|global_store|buffer_store)\w*")
_LDS_DMA = re.compile(r"^\s*global_load_lds|^\s*buffer_load\w*.*\blds\b")


def _regs(text):
    out = set()
    for m in _SREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _operands(line):
    body = line.split(";")[0].strip()
    parts = body.split(None, 1)
    return parts[0], (parts[1] if len(parts) > 1 else "")


def _valu_sgpr_defs(mnem, ops):
    """SGPRs a VALU instruction may write: the scalar destinations among its
    first two operands (v_readlane/v_readfirstlane, VOP3 compares and
    carry-outs)."""
    if not mnem.startswith("v_"):
        return set()
    first = [o.strip() for o in ops.split(",")[:2]]
    if mnem.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
        return _regs(first[0]) if first else set()
    if mnem.endswith("_e64") and len(first) > 1 and ("co_" in mnem or "div_scale" in mnem):
        return _regs(first[1])
    return set()


def _wait_states(mnem, ops):
    if mnem == "s_nop":
        try:
            return int(ops.strip(), 0) + 1
        except ValueError:
            return 1
    return 1


_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
MFMA_VGPR_READ_WAIT = 11


def _vregs(text):
    out = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _scan_mfma_results(lines, findings):
    """Inline-asm MFMAs with a VGPR destination: the first later instruction
    that touches the destination must come MFMA_VGPR_READ_WAIT wait states
    later, unless it is an MFMA accumulating into the same registers."""
    in_asm = False
    for i, raw in enumerate(lines):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not in_asm or not s.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        if not ops[0].startswith("v"):
            continue                                  # AGPR destination: tracked by the compiler
        dst = _vregs(ops[0])
        ws = 0
        for j in range(i + 1, min(len(lines), i + 200)):
            p = lines[j].strip()
            if not p or p.startswith(";") or p.startswith("."):
                if p.endswith(":"):
                    break                             # a label: other paths are checked on their own
                continue
            if p.endswith(":"):
                break
            pm, po = _operands(p)
            if pm.startswith("v_mfma"):
                pops = [o.strip() for o in po.split(",")]
                if _vregs(pops[0]) == dst and len(pops) > 3 and _vregs(pops[3]) == dst:
                    break                             # the chain's next step (forwarded)
                if dst & _vregs(",".join(pops[1:])):
                    findings.append((j + 1, p, f"MFMA result read as an operand {ws} wait states after "
                                               f"line {i + 1}"))
                    break
                ws += 1
                continue
            if dst & _vregs(po):
                if ws < MFMA_VGPR_READ_WAIT:
                    findings.append((j + 1, p, f"MFMA result (line {i + 1}) touched {ws} wait states after it"))
                break
            ws += _wait_states(pm, po)
            if ws >= MFMA_VGPR_READ_WAIT:
                break


def scan(asm_text):
    """Return a list of (line number, instruction, reason) hazard findings."""
    lines = asm_text.splitlines()
    findings = []
    _scan_mfma_results(lines, findings)
    in_asm = False
    for i, raw in enumerate(lines):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not in_asm or not s or s.startswith(";"):
            continue
        mnem, ops = _operands(s)
        if not _VMEM.match(s):
            continue
        # scalar registers this memory instruction reads (its base address)
        sregs = _regs(ops)
        need_m0 = bool(_LDS_DMA.match(s))
        # wait states inside the same asm block before this instruction
        ws = 0
        j = i - 1
        inside = True
        while j >= 0:
            p = lines[j].strip()
            if p.startswith(";;#ASMSTART"):
                inside = False
                j -= 1
                continue
            if p.startswith(";;#ASMEND"):
                j -= 1
                continue
            if not p or p.startswith(";") or p.startswith("."):
                if p.endswith(":"):      # a label: another block may enter here
                    break
                j -= 1
                continue
            if p.endswith(":"):
                break
            pm, po = _operands(p)
            defs = _valu_sgpr_defs(pm, po)
            if sregs & defs and ws < 5:
                findings.append((i + 1, s, f"VALU writes {sorted(sregs & defs)} {ws} wait states before "
                                           f"({lines[j].strip()})"))
                break
            if need_m0 and ws < 1 and re.match(r"^s_\w+\s+m0\b", p):
                findings.append((i + 1, s, f"M0 written {ws} wait states before ({p})"))
            ws += _wait_states(pm, po)
            if ws >= 5 and not inside:
                break
            j -= 1
    return findings
