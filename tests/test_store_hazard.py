"""Host-side check of the compiled stage-1 code for an open wide-store hazard.

A buffer store of more than 8 bytes reads its data registers after it issues,
so the next two wait states must not rewrite them.  The compiler inserts that
wait only when the store's scalar offset is not a register; stage 1 therefore
passes every record offset in the vector offset.  This test compiles the
stage-1 kernel and the fused chain-and-stage-1 kernel for gfx950 to assembly
and fails if any 12- or 16-byte buffer store has a data register written by a
vector, LDS or memory instruction within the two wait states after it.  No GPU
is needed.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_07_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
WAIT_STATES = 2


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def open_wide_stores(asm_lines):
    """(store, next instruction) pairs where the next WAIT_STATES wait states rewrite store data."""
    hits, nstores = [], 0
    for i, line in enumerate(asm_lines):
        m = re.match(r"buffer_store_dwordx[34]\s+(v\[\d+:\d+\]),", line)
        if not m:
            continue
        nstores += 1
        data = _vregs(m.group(1))
        ws, j = 0, i + 1
        while ws < WAIT_STATES and j < len(asm_lines):
            nxt = asm_lines[j]
            j += 1
            if not nxt or nxt.startswith((";", ".")) or nxt.endswith(":"):
                continue
            if nxt.startswith("s_nop"):
                ws += int(nxt.split()[1]) + 1
                continue
            ws += 1
            op = nxt.split()[0]
            if op.startswith(("v_", "ds_read", "buffer_load", "global_load")):
                if _vregs(nxt.split()[1].rstrip(",")) & data:
                    hits.append((line, nxt))
    return nstores, hits


def test_scanner_flags_a_rewrite():
    lines = ["buffer_store_dwordx4 v[2:5], v0, s[16:19], s0 offen", "v_lshl_add_u32 v2, v18, 2, s24"]
    assert open_wide_stores(lines) == (1, [(lines[0], lines[1])])
    lines = ["buffer_store_dwordx4 v[2:5], v0, s[16:19], 0 offen", "s_nop 1", "v_lshl_add_u32 v2, v18, 2, s24"]
    assert open_wide_stores(lines) == (1, [])


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
@pytest.mark.parametrize("src", ["kda_prep.hip", "kda_prefill_pipe.hip"])
def test_no_open_wide_store(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    lines = [ln.strip() for ln in out.read_text().splitlines()]
    nstores, hits = open_wide_stores(lines)
    assert nstores > 0
    assert not hits, hits[:5]
