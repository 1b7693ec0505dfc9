"""Static checks of the grouped-GEMM kernels' gfx950 assembly (CPU only; needs hipcc).

The MFMAs of the K loop are inline asm, so the compiler neither pads them for hazards nor
checks their operands. These tests compile gemm.hip to assembly and check what the
kernel's construction promises:
  * no VALU instruction writes a VGPR that an MFMA reads (A, B or a scale word) within
    the 2 wait states such a write needs before an MFMA may read it;
  * the accumulators stay in place: every MFMA's destination equals its accumulator input
    and the K loops move no accumulator (no v_accvgpr_read / write / mov inside a loop);
  * every read of an accumulator comes at least 19 wait states after the MFMA that last
    wrote it (the most a 16x16 MFMA's result needs before a VALU may read it), counting
    every instruction in between, MFMAs included, as one and s_nop N as N + 1;
  * the kernels use no scratch memory inside their K loops.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp8_dispatch_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", os.path.join(CSRC, "gemm.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return [l.strip() for l in open(out)]


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _is_instr(line):
    return bool(line) and not line.startswith((";", ".", "#")) and not line.endswith(":")


def _mfma_operands(line):
    ops = [o.strip().split()[0] for o in line.split(None, 1)[1].split(",")]
    return ops   # dst, A, B, C, scale A, scale B


def test_no_valu_write_of_an_mfma_source_within_two_wait_states(asm):
    checked = 0
    for i, line in enumerate(asm):
        if not line.startswith("v_mfma"):
            continue
        ops = _mfma_operands(line)
        src = _vregs(ops[1]) | _vregs(ops[2]) | _vregs(ops[4]) | _vregs(ops[5])
        waits, j = 0, i - 1
        while j >= 0 and waits < 2:
            p = asm[j]
            j -= 1
            if not _is_instr(p):
                continue
            op = p.split()[0]
            if op.startswith("v_") and not op.startswith("v_mfma"):
                dst = p.split(None, 1)[1].split(",")[0].strip()
                assert not (_vregs(dst) & src), f"VALU write {p!r} {waits} wait states before {line!r}"
            waits += int(p.split()[1]) + 1 if op == "s_nop" else 1
        checked += 1
    assert checked > 1000


def _loops(asm):
    """(start, end) line ranges of every innermost loop (header label .. backward branch)."""
    out = []
    for i, line in enumerate(asm):
        if "Inner Loop Header" in line:
            # the marker follows the block label, on its line or on the next one
            j = i
            while j > 0 and not asm[j].split(";")[0].strip().endswith(":"):
                j -= 1
            label = asm[j].split(":")[0]
            for j in range(i + 1, len(asm)):
                if asm[j].startswith("s_cbranch") and asm[j].split()[-1] == label:
                    out.append((i, j))
                    break
    return out


def test_accumulators_stay_tied_and_in_place(asm):
    n_mfma_loops = 0
    for a, b in _loops(asm):
        body = [l for l in asm[a:b + 1] if _is_instr(l)]
        mfmas = [l for l in body if l.startswith("v_mfma")]
        if not mfmas:
            continue
        n_mfma_loops += 1
        for l in mfmas:
            ops = _mfma_operands(l)
            assert ops[0] == ops[3] and ops[0].startswith("a["), l
        moves = [l for l in body if l.startswith(("v_accvgpr_read", "v_accvgpr_write", "v_accvgpr_mov"))]
        assert not moves, moves[:4]
        assert not [l for l in body if l.startswith("scratch_")]
    # Linear1 (A blocked or through the row list), Linear2 (32- or 64-bit stage offsets),
    # plain GEMM: three row-tile classes each, and a 128-row second-launch kernel each (with
    # non-temporal B loads); split-K: two
    assert n_mfma_loops == 22


def _aregs(tok):
    m = re.match(r"a\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def test_accumulator_reads_wait_for_their_mfma(asm):
    checked = 0
    for i, line in enumerate(asm):
        if not line.startswith("v_accvgpr_read"):
            continue
        src = _aregs(line.split(None, 1)[1].split(",")[1].strip())
        waits, j = 0, i - 1
        while j >= 0 and waits < 19:
            p = asm[j]
            j -= 1
            if p.startswith(".Lfunc_end") or p.startswith(".amdhsa_kernel"):
                break
            if not _is_instr(p):
                continue
            if p.startswith("v_mfma"):
                assert not (_aregs(_mfma_operands(p)[0]) & src), \
                    f"{line!r} only {waits} wait states after {p!r}"
            waits += int(p.split()[1]) + 1 if p.split()[0] == "s_nop" else 1
        checked += 1
    assert checked > 1000
