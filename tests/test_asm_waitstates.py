"""Host-side checks of the generated gfx950 code of the sparse MLA kernels (no GPU
needed): the parts the compiler cannot see are written by hand, so the
generated code is checked for them.

* The O^T += V^T P^T MFMAs are inline assembly; the compiler inserts no wait
  states before them.  No VALU instruction may write one of their source
  registers within the few instructions before them unless enough s_nop wait
  states separate the two.
* m0 (the LDS base of the global -> LDS copies) is set only inside the copy's
  own assembly, so nothing else in the kernels relies on its value.
"""
import os
import re
import shutil
import subprocess

import pytest

from long_context_sparse_fp8_amd import build as B

MFMA_ASM = re.compile(r"v_mfma_f32_32x32x16_bf16 a\[\d+:\d+\], v\[(\d+):(\d+)\], v\[(\d+):(\d+)\]")
VALU_DST = re.compile(r"^(v_\S+)\s+(?:v(\d+)|v\[(\d+):(\d+)\])")
NEED_WAIT_STATES = 5     # VALU write of a VGPR -> MFMA read of it as SrcA/SrcB (conservative)
LOOKBACK = 8             # instructions inspected before each asm MFMA


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "sparse_mla.s"
    cmd = [B.HIPCC, *B.FLAGS, *B.SOURCE_FLAGS.get("sparse_mla.hip", []), "-x", "hip", "-S", "--cuda-device-only",
           os.path.join(B.CSRC, "sparse_mla.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def _instructions_before(lines, idx, n):
    """Up to n instructions before line idx (comments, labels and asm markers skipped)."""
    out, k = [], idx - 1
    while k >= 0 and len(out) < n:
        t = lines[k].strip()
        if t and not t.startswith(";") and not t.startswith("."):
            out.append(t)
        k -= 1
    return out


def test_asm_mfma_operands_not_written_just_before(asm):
    n_mfma = 0
    for idx, line in enumerate(asm):
        m = MFMA_ASM.search(line)
        if not m:
            continue
        n_mfma += 1
        regs = set(range(int(m.group(1)), int(m.group(2)) + 1)) | set(range(int(m.group(3)), int(m.group(4)) + 1))
        waits = 0
        for ins in _instructions_before(asm, idx, LOOKBACK):
            op = ins.split()[0]
            if op == "s_nop":
                waits += int(ins.split()[1]) + 1
                continue
            d = VALU_DST.match(ins)
            if d and not op.startswith("v_mfma"):
                dst = {int(d.group(2))} if d.group(2) else set(range(int(d.group(3)), int(d.group(4)) + 1))
                assert not (dst & regs) or waits >= NEED_WAIT_STATES, (idx, ins, line.strip())
    assert n_mfma > 0, "no O^T MFMAs found: the pattern is out of date"


def test_m0_written_only_by_the_copies(asm):
    inside = False
    n_copies = 0
    for line in asm:
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
        elif t.startswith(";;#ASMEND"):
            inside = False
        elif re.match(r"^s_\S+\s+m0\b", t):
            assert inside, t
        if "global_load_lds_dwordx4" in t:
            n_copies += 1
    assert n_copies > 0
