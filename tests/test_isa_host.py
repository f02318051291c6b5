"""Host-side check of the gfx950 code the decode source compiles to (no GPU).

The packed fp6 conversions that build the query operand (v_cvt_scalef32_2xpk16_fp6_f32 and
v_cvt_scalef32_pk32_f32_fp6) read their sources after writing part of their destination, while the
compiler is free to give the destination registers that a source still occupies when that source dies
at the instruction; the values in the overlapped registers then come out wrong.  The source keeps every
operand live across each conversion; this test compiles it with the library's own flags and checks that
no conversion's destination overlaps one of its operands.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "bit_kv_cache_qjl_amd"))
import build as qbuild  # noqa: E402  (the package's build script; importing it builds nothing)

CONV = re.compile(r"\b(v_cvt_scalef32_(?:2xpk16_fp6_f32|pk32_f32_fp6))\s+v\[(\d+):(\d+)\],\s*(.*)$")


def _regs(operands: str) -> set:
    regs = set()
    for lo, hi in re.findall(r"v\[(\d+):(\d+)\]", operands):
        regs |= set(range(int(lo), int(hi) + 1))
    for r in re.findall(r"(?<![\[\d:])v(\d+)\b", operands):
        regs.add(int(r))
    return regs


def overlapping_conversions(asm: str) -> tuple[int, list]:
    n, bad = 0, []
    for line in asm.splitlines():
        m = CONV.search(line)
        if not m:
            continue
        n += 1
        dst = set(range(int(m.group(2)), int(m.group(3)) + 1))
        if dst & _regs(m.group(4)):
            bad.append(line.strip())
    return n, bad


def test_scanner_flags_an_overlap():
    n, bad = overlapping_conversions("\tv_cvt_scalef32_2xpk16_fp6_f32 v[32:37], v[2:17], v[18:33], s0\n"
                                     "\tv_cvt_scalef32_2xpk16_fp6_f32 v[16:21], v[0:15], v[32:47], v16\n"
                                     "\tv_cvt_scalef32_pk32_f32_fp6 v[0:31], v[64:69], v107\n")
    assert n == 3 and len(bad) == 2


@pytest.mark.skipif(not os.path.exists(qbuild.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_fp6_conversions_never_overwrite_their_operands(tmp_path):
    src = "qjl_decode_mfma.hip"
    out = tmp_path / "decode.s"
    cmd = [qbuild.HIPCC, *[f for f in qbuild.FLAGS if f != "-fPIC"], *qbuild.EXTRA.get(src, []),
           "--offload-device-only", "-S", os.path.join(qbuild.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    n, bad = overlapping_conversions(out.read_text())
    assert n > 0, "the query operand no longer uses the packed fp6 conversions"
    assert not bad, "conversion destination overlaps an operand:\n" + "\n".join(bad[:10])
