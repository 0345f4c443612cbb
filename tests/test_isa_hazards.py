"""The kernels' hand-placed MFMA hazard guards, checked on the compiled gfx950
assembly (CPU only: hipcc cross-compiles, nothing runs on a GPU).

Many MFMAs are inline asm with fixed register classes, which the compiler's
hazard recognizer does not see, so the wait states between an MFMA and the
VALU work that reads its results (and between a VALU write and an MFMA that
reads it) are kept by hand.  A missing guard gives wrong numbers with no
error, only now and then; this test compiles every HIP source to assembly
with the library's own flags and scans each kernel (tests/isa_hazards.py).
"""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_attention_33_amd import build as B
from tests import isa_hazards

HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def test_scan_catches_planted_hazards():
    """The scan is not vacuous: an MFMA result read 8 wait states after the
    MFMA (11 needed) and an MFMA operand written by the VALU right before it
    are both reported; with the guards in place nothing is."""
    bad = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
           "s_nop 7",
           "v_add_f32_e32 v30, v1, v2",
           "v_mov_b32_e32 v16, v3",
           "v_mfma_f32_32x32x16_bf16 v[40:55], v[16:19], v[20:23], 0"]
    found = isa_hazards.scan(bad)
    assert {(f[0], f[2]) for f in found} >= {(2, ("v", 1)), (2, ("v", 2)), (4, ("v", 16))}
    good = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
            "s_nop 7", "s_nop 2",
            "v_add_f32_e32 v30, v1, v2",
            "v_mov_b32_e32 v16, v3",
            "s_nop 1",
            "v_mfma_f32_32x32x16_bf16 v[40:55], v[16:19], v[20:23], 0"]
    assert isa_hazards.scan(good) == []
    # an MFMA at a branch target: the branch counts one wait state, so the
    # instruction ahead of each branch to the label is checked too
    mf = "v_mfma_f32_32x32x16_bf16 v[40:55], v[16:19], v[20:23], 0"
    tgt = ["v_mov_b32_e32 v17, v3", "s_cbranch_scc1 .L1", "s_nop 7", "<label> .L1", mf]
    assert [f[2] for f in isa_hazards.scan(tgt)] == ["branch target"]
    assert isa_hazards.scan(["v_mov_b32_e32 v99, v3"] + tgt[1:]) == []
    assert isa_hazards.scan(tgt[:4] + ["s_waitcnt lgkmcnt(0)", mf]) == []   # branch + 1
    ks = isa_hazards.kernels("_Zk:\n  s_nop 0\n.LBB0_1:\n  .p2align 6\n  s_endpgm\n")
    assert ks["_Zk"] == ["s_nop 0", "<label> .LBB0_1", "s_endpgm"]
    # a 16-pass (fp8) MFMA needs 19
    fp8 = ["v_mfma_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], 0", "s_nop 7", "s_nop 7",
           "v_add_f32_e32 v30, v1, v2"]
    assert [f[4] for f in isa_hazards.scan(fp8)] == [19, 19]


def _hipcc():
    return B.hipcc()


@pytest.mark.skipif(not os.path.exists(_hipcc()), reason="hipcc not installed")
def test_every_kernel_keeps_its_mfma_wait_states():
    tmp = tempfile.mkdtemp(prefix="fa_isa_")
    try:
        flags = [f for f in B.FLAGS if f != "-fPIC"]

        def compile_one(src):
            out = os.path.join(tmp, os.path.splitext(src)[0] + ".s")
            r = subprocess.run([_hipcc(), "-x", "hip", *flags, "--cuda-device-only", "-S",
                                os.path.join(B.CSRC, src), "-o", out],
                               stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
            assert r.returncode == 0, r.stdout[-2000:]
            return src, out

        with ThreadPoolExecutor(max_workers=min(8, len(HIP_SOURCES))) as ex:
            outs = list(ex.map(compile_one, HIP_SOURCES))
        report, n_kernels, n_mfma = [], 0, 0
        for src, path in outs:
            with open(path) as f:
                ks = isa_hazards.kernels(f.read())
            for name, lines in ks.items():
                n_kernels += 1
                n_mfma += sum("mfma" in l for l in lines)
                for i, op, reg, seen, need in isa_hazards.scan(lines):
                    report.append(f"{src} {name[:90]} instr {i} {op} {reg}: {seen} wait states, {need} needed")
        assert n_kernels > 40 and n_mfma > 1000, (n_kernels, n_mfma)
        assert not report, "\n".join(report[:40])
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
