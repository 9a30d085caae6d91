"""MFMA result reads and wait states, checked on the compiled gfx950 code.

A VALU instruction that reads a VGPR written by an MFMA needs a number of
wait states first; the hardware does not stall for it, the compiler pads
with s_nop.  Inside a basic block the compiler pads these reads to 8 wait
states.  A read reached through a branch right after the MFMA once got only
4 and silently used stale accumulators (wrong router scores).  This test
builds each kernel source to assembly with the library's flags and walks
every control-flow path from every MFMA to the first instruction reading its
result, asserting at least 8 wait states on each path.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_sparse_long_key_amd import build as libbuild  # noqa: E402

NEED = 8
SOURCES = ["router.hip", "attn.hip", "attn_bwd.hip"]


def _regs(op):
    op = op.replace("|", "").lstrip("-")
    m = re.match(r"v\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


def _functions(asm):
    for name, body in re.findall(r"^(_Z\S+):[^\n]*\n(.*?)\.Lfunc_end", asm, re.M | re.S):
        lines = [l.split(";")[0].strip() for l in body.splitlines()]
        lines = [l for l in lines if l and not l.startswith(".") or re.match(r"^\.LBB\S+:$", l or "")]
        labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}
        yield name, lines, labels


def _first_reads(lines, labels, start, dst, ws, seen):
    """(wait states, instruction) of the first read of dst on each path."""
    out = []
    i = start
    while i < len(lines) and ws < NEED:
        line = lines[i]
        i += 1
        if line.endswith(":"):
            continue
        op = line.split()[0]
        args = [a.strip() for a in line[len(op):].split(",")]
        if not op.startswith("s_") and not op.startswith("v_mfma"):
            stores = op.startswith(("global_store", "ds_write", "buffer_store", "flat_store"))
            read = set()
            for a in (args if stores else args[1:]):
                read |= _regs(a)
            if read & dst:
                out.append((ws, line))
                return out
        ws += int(args[0], 0) + 1 if op == "s_nop" else 1
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = args[0]
            if tgt in labels and (tgt, ws) not in seen:
                seen.add((tgt, ws))
                out += _first_reads(lines, labels, labels[tgt] + 1, dst, ws, seen)
            if op == "s_branch":
                return out
        if op == "s_endpgm":
            return out
    return out


@pytest.mark.skipif(shutil.which(libbuild.HIPCC) is None and not os.path.exists(libbuild.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("debug", [False, True], ids=["release", "debug-bounds"])
@pytest.mark.parametrize("src", SOURCES)
def test_mfma_results_read_after_enough_wait_states(src, debug, tmp_path):
    """Both builds: the bounds-checking one adds branches of its own."""
    out = tmp_path / (src + ".s")
    cmd = [libbuild.HIPCC, *libbuild.FLAGS, *(["-DMOBA_DEBUG_BOUNDS"] if debug else []),
           "--cuda-device-only", "-S", os.path.join(libbuild.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    bad = []
    nmfma = 0
    for name, lines, labels in _functions(asm):
        for i, line in enumerate(lines):
            if not line.startswith("v_mfma"):
                continue
            nmfma += 1
            dst = _regs(line.split(None, 1)[1].split(",")[0].strip())
            for ws, instr in _first_reads(lines, labels, i + 1, dst, 0, set()):
                bad.append(f"{name[:70]}: {ws} wait states before `{instr}` after `{line}`")
    assert nmfma > 0
    assert not bad, "\n".join(bad[:20])
