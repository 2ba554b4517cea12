"""Wait states before the direct global->LDS loads, checked on the generated gfx950 assembly.

The kernels issue ``global_load_lds_dwordx4`` from inline assembly.  The load reads
M0 (its LDS address) and, in the SADDR form, a 64-bit base in an SGPR pair.  When a
vector instruction (for example a lane read, ``v_readfirstlane_b32``) writes one of
those SGPRs, the hardware needs five wait states before a memory instruction reads
it, and the compiler does not insert them for assembly it cannot see into; a load
issued too early uses a stale address.  This test compiles every attention source
with the library's own flags to assembly (host-only, no GPU) and checks that each
such load is at least five wait states behind the last vector write of every SGPR
it reads (``s_nop N`` counts N+1, any other instruction one).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from fp8_attention_amd import build

SOURCES = [s for s in build.SOURCES if s.startswith("attn_")]
LOAD = "global_load_lds_dwordx4"


def _assembly(src: str, outdir: str) -> str:
    out = os.path.join(outdir, os.path.splitext(src)[0] + ".s")
    cmd = [build.HIPCC, *build.FLAGS, *build.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc -S failed on {src}:\n{r.stderr[-2000:]}"
    return out


def _sgprs_read(line: str) -> list:
    regs = ["m0"]
    m = re.search(r"s\[(\d+):(\d+)\]", line)
    if m:
        regs += [int(m.group(1)), int(m.group(2))]
    return regs


def _writes(instr: str, reg) -> bool:
    """Does this instruction write SGPR reg (an int) or M0?"""
    parts = instr.replace(",", " ").split()
    if len(parts) < 2:
        return False
    dst = parts[1]
    if reg == "m0":
        return dst == "m0"
    if dst == f"s{reg}":
        return True
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", dst)
    return bool(m) and int(m.group(1)) <= reg <= int(m.group(2))


def hazards(asm_text: str) -> list:
    """(line number, register, distance) for every load read too soon after a vector write."""
    lines = [l.split(";")[0].strip() for l in asm_text.split("\n")]
    found = []
    for i, line in enumerate(lines):
        if not line.startswith(LOAD):
            continue
        for reg in _sgprs_read(line):
            dist = 0
            for k in range(i - 1, max(-1, i - 200), -1):
                x = lines[k]
                if not x or x.startswith(".") or x.endswith(":"):
                    continue                     # labels and directives: scan on along the fall-through path
                if x.startswith("s_nop"):
                    dist += int(x.split()[1], 0) + 1
                    continue
                if _writes(x, reg):
                    if x.startswith("v_") and dist < 5:
                        found.append((i + 1, reg, dist))
                    break
                dist += 1
                if dist >= 5:
                    break
    return found


def test_hazard_scan_finds_a_planted_case():
    # a lane read that writes the load's base right before it is a hazard; five nops are not
    bad = "v_readfirstlane_b32 s4, v1\nv_readfirstlane_b32 s5, v2\ns_nop 0\nglobal_load_lds_dwordx4 v3, s[4:5]\n"
    good = "v_readfirstlane_b32 s4, v1\nv_readfirstlane_b32 s5, v2\ns_nop 4\nglobal_load_lds_dwordx4 v3, s[4:5]\n"
    salu = "s_add_u32 s4, s6, s8\ns_addc_u32 s5, s7, 0\ns_nop 0\nglobal_load_lds_dwordx4 v3, s[4:5]\n"
    m0 = "v_readfirstlane_b32 m0, v9\ns_nop 0\nglobal_load_lds_dwordx4 v[2:3], off\n"
    assert [(r, d) for _, r, d in hazards(bad)] == [(4, 2), (5, 1)]
    assert hazards(good) == []
    assert hazards(salu) == []
    assert [(r, d) for _, r, d in hazards(m0)] == [("m0", 1)]


@pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC), reason="hipcc not found")
def test_direct_loads_wait_for_vector_written_sgprs():
    with tempfile.TemporaryDirectory() as d:
        with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
            outs = list(ex.map(lambda s: _assembly(s, d), SOURCES))
        bad = {}
        nloads = 0
        for src, out in zip(SOURCES, outs):
            text = open(out).read()
            nloads += text.count(LOAD)
            h = hazards(text)
            if h:
                bad[src] = h[:5]
    assert nloads > 0
    assert not bad, f"direct loads too close to a vector write of their SGPR operands: {bad}"
