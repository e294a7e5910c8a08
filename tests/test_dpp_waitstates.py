"""The hand-written DPP multiply-adds of the UT substitution keep gfx9's wait-state rule.

A DPP instruction may not read a VGPR that a vector ALU instruction wrote in the two instructions before it;
the compiler inserts those wait states for the instructions it emits itself, not for inline assembly.  This
compiles every source that uses the row broadcast to gfx950 device assembly and checks each DPP instruction
against the instructions before it (an ``s_nop N`` counts as N + 1 wait states, any other instruction as one).
"""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from exact_flow_delta_amd import build as B

_VREG = re.compile(r"^-?\|?v(?:\[(\d+):(\d+)\]|(\d+))")


def _vregs(tok):
    m = _VREG.match(tok.strip())
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def dpp_hazards(asm_lines):
    """(number of DPP instructions, list of offending lines) for one assembly listing."""
    recent = []   # (wait states since, VGPRs written) of the last instructions, newest last
    n_dpp, bad = 0, []
    for ln in asm_lines:
        s = ln.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        op = s.split()[0]
        args = [a for a in (x.strip() for x in s[len(op):].split(",")) if a]
        if op == "s_nop":
            n = int(args[0], 0) + 1
            recent = [(w + n, r) for w, r in recent]
            continue
        if "_dpp" in op:
            n_dpp += 1
            used = set()
            for a in args:
                used |= _vregs(a.split()[0])
            if any(w < 2 and (r & used) for w, r in recent):
                bad.append(s)
        written = _vregs(args[0]) if op.startswith("v_") and args else set()
        recent = [(w + 1, r) for w, r in recent if w + 1 < 2] + [(0, written)]
    return n_dpp, bad


def test_scanner_flags_a_fresh_write():
    lines = ["v_mov_b32_e32 v3, v1", "v_fmac_f32_dpp v2, -v3, v4 row_newbcast:1 row_mask:0xf bank_mask:0xf"]
    assert dpp_hazards(lines) == (1, [lines[1]])
    assert dpp_hazards([lines[0], "s_nop 1", lines[1]]) == (1, [])
    assert dpp_hazards([lines[0], "v_add_f32_e32 v7, v8, v9", "v_mul_f32_e32 v5, v6, v6", lines[1]]) == (1, [])


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC), reason="hipcc not found")
def test_row_broadcast_multiply_adds_keep_wait_states(tmp_path):
    srcs = [s for s in B.SOURCES if _uses_row_bcast(s)]
    assert srcs, "no source uses the row broadcast"

    def compile_asm(src):
        out = tmp_path / (src + ".s")
        cmd = [B.HIPCC] + [f for f in B.CFLAGS if f != "-fPIC"] + ["--cuda-device-only", "-S",
                                                                   os.path.join(B.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return src, out

    total = 0
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        for src, out in ex.map(compile_asm, srcs):
            n, bad = dpp_hazards(out.read_text().splitlines())
            total += n
            assert not bad, "%s: DPP reads a fresh VGPR: %s" % (src, bad[:3])
    assert total > 0


def _uses_row_bcast(src):
    """A source uses the row broadcast if it includes, at any depth, a file that calls tri_solve_row_bcast."""
    users = [f for f in os.listdir(B.CSRC) if f != "efla_common.hpp" and f.endswith((".hpp", ".hip"))
             and "tri_solve_row_bcast<" in open(os.path.join(B.CSRC, f)).read()]
    seen, todo = set(), [src]
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        path = os.path.join(B.CSRC, f)
        if not os.path.exists(path):   # the public header and system headers
            continue
        text = open(path).read()
        if f in users:
            return True
        todo += re.findall(r'#include "([^"]+)"', text)
    return False
