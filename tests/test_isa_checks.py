"""Checks on the gfx950 assembly the kernels compile to (CPU only).

A 128-bit buffer store whose scalar offset is a register, followed at once
by a VALU write of one of the store's data registers, lost that dword to the
new value on the hardware: a few output elements came out different from run
to run.  The compiler keeps the data registers untouched for the needed wait
state only when the scalar offset is a constant, so every buffer store in the
kernels folds its whole offset into the per-lane offset.  This test compiles
every HIP source to assembly and fails if a wide store with a register
scalar offset appears again.

It also checks the MFMA operand rule the compiler enforces for wide results
(a destination wider than four registers must not partially overlap the
accumulator input), in case an inline-asm path ever bypasses it.
"""
import concurrent.futures
import os
import re

import subprocess

import pytest

from linear_rnn_lm_amd import build as B

REG = re.compile(r"([vas])\[(\d+):(\d+)\]|([vas])(\d+)")


def _regs(op):
    m = REG.fullmatch(op.strip())
    if not m:
        return None
    if m.group(1):
        return m.group(1), int(m.group(2)), int(m.group(3))
    return m.group(4), int(m.group(5)), int(m.group(5))


def wide_stores_with_register_soffset(asm_text):
    """buffer_store_dwordx3/x4 lines whose scalar offset operand is an SGPR."""
    bad = []
    for line in asm_text.splitlines():
        s = line.strip()
        if not (s.startswith("buffer_store_dwordx4") or s.startswith("buffer_store_dwordx3")):
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        # vdata, vaddr, srsrc, soffset [modifiers]
        soff = ops[3].split()[0] if len(ops) > 3 else ""
        r = _regs(soff)
        if r and r[0] == "s":
            bad.append(s)
    return bad


def wide_mfma_partial_overlaps(asm_text):
    """MFMAs with more than four destination registers that partially overlap srcC."""
    bad = []
    for line in asm_text.splitlines():
        s = line.strip()
        if not s.startswith("v_mfma"):
            continue
        ops = s.split(None, 1)[1].split(",")
        if len(ops) < 4:
            continue
        d, c = _regs(ops[0]), _regs(ops[3])
        if not (d and c) or d[2] - d[1] + 1 <= 4:
            continue
        if d[0] == c[0] and d != c and not (d[2] < c[1] or c[2] < d[1]):
            bad.append(s)
    return bad


def _asm(src, tmp):
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "-S", "--cuda-device-only", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    with open(out) as f:
        return f.read()


def test_detectors_on_examples():
    assert wide_stores_with_register_soffset("\tbuffer_store_dwordx4 v[16:19], v28, s[44:47], s0 offen")
    assert not wide_stores_with_register_soffset("\tbuffer_store_dwordx4 v[16:19], v28, s[44:47], 0 offen")
    assert not wide_stores_with_register_soffset("\tbuffer_store_dword v16, v28, s[44:47], s0 offen")
    assert wide_mfma_partial_overlaps("\tv_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[8:23]")
    assert not wide_mfma_partial_overlaps("\tv_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]")
    assert not wide_mfma_partial_overlaps("\tv_mfma_f32_16x16x32_bf16 v[12:15], v[56:59], v[18:21], v[14:17]")


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    tmp = str(tmp_path_factory.mktemp("asm"))
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        return list(ex.map(lambda s: _asm(s, tmp), srcs))


def test_wide_buffer_stores_use_constant_scalar_offset(kernel_asm):
    n = sum(t.count("buffer_store_dwordx4") for t in kernel_asm)
    assert n > 0
    bad = [b for t in kernel_asm for b in wide_stores_with_register_soffset(t)]
    assert not bad, bad[:5]


def test_no_wide_mfma_with_partially_overlapping_accumulator(kernel_asm):
    assert sum(t.count("v_mfma") for t in kernel_asm) > 1000
    bad = [b for t in kernel_asm for b in wide_mfma_partial_overlaps(t)]
    assert not bad, bad[:5]
