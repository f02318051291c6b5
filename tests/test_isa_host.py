"""Host-side checks of the gfx950 code the decode source compiles to (no GPU).

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


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    """The decode source compiled to gfx950 assembly with the library's flags (once per module)."""
    if not os.path.exists(qbuild.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    src = "qjl_decode_mfma.hip"
    out = tmp_path_factory.mktemp("isa") / "decode.s"
    cmd = [qbuild.HIPCC, *[f for f in qbuild.FLAGS if f != "-fPIC"], *qbuild.EXTRA.get(src, []),
           "--offload-device-only", "-S", os.path.join(qbuild.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_fp6_conversions_never_overwrite_their_operands(decode_asm):
    n, bad = overlapping_conversions(decode_asm)
    assert n > 0, "the query operand no longer uses the packed fp6 conversions"
    assert not bad, "conversion destination overlaps an operand:\n" + "\n".join(bad[:10])


def _kernel_asm(asm: str, symbol_prefix: str) -> str:
    start = asm.index("\n" + symbol_prefix)
    return asm[start:asm.index("s_endpgm", start)]


def block_loop(kernel_asm: str, marker: str = "") -> str:
    """The body of the kernel's last loop that contains `marker` (from its header label to the branch
    back to it; with no marker, the last loop)."""
    headers = re.findall(r"^(\.LBB\w+):.*Loop Header", kernel_asm, re.M)
    assert headers, "no loop found"
    for label in reversed(headers):
        body = kernel_asm[kernel_asm.index(label + ":"):]
        body = body[:body.rindex(label)]
        if marker in body:
            return body
    return ""


def test_block_loop_finds_the_last_loop():
    fake = ("\nk:\n\ts_mov_b32 s0, 0\n.LBB0_1:  ; =>This Inner Loop Header: Depth=1\n\ts_waitcnt vmcnt(3)\n"
            "\ts_cbranch_scc1 .LBB0_1\n.LBB0_2:  ; =>This Inner Loop Header: Depth=1\n\ts_waitcnt vmcnt(0)\n"
            "\tbuffer_load_dword v0, s[0:3], 0 offen lds\n\ts_cbranch_scc1 .LBB0_2\n\ts_endpgm\n")
    loop = block_loop(_kernel_asm(fake, "k:"))
    assert re.findall(r"s_waitcnt vmcnt\((\d+)\)", loop) == ["0"]


def test_eight_wave_block_loop_waits_only_where_written(decode_asm):
    """The eight-wave decode's block loop waits for its buffer loads only with the explicit counts the
    source writes: the compiler cannot tell its LDS buffers apart, and a wait for every outstanding load
    (vmcnt(0)) inserted before an LDS access it sees would also wait for the next block's code loads,
    issued just before."""
    asm = decode_asm
    # both sketch widths, with the query projection in the kernel (Lb1E) and after a projection launch (Lb0E)
    for sym in ("_ZN3qjl12_GLOBAL__N_119decode_mfma8_kernelILi2ELi2ELb0ELb1E", "_ZN3qjl12_GLOBAL__N_119decode_mfma8_kernelILi4ELi0ELb0ELb1E",
                "_ZN3qjl12_GLOBAL__N_119decode_mfma8_kernelILi2ELi2ELb0ELb0E", "_ZN3qjl12_GLOBAL__N_119decode_mfma8_kernelILi4ELi0ELb0ELb0E"):
        loop = block_loop(_kernel_asm(asm, sym), "v_mfma_scale_f32_16x16x128_f8f6f4")
        assert "v_mfma_scale_f32_16x16x128_f8f6f4" in loop and "lds" in loop, "not the block loop"
        waits = re.findall(r"s_waitcnt vmcnt\((\d+)\)", loop)
        assert waits and "0" not in waits, f"{sym}: vmcnt waits in the block loop: {waits}"
