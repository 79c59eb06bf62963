"""Static checks of the gfx950 code the kernels compile to.

Matrix (MFMA) instructions do not honour the EXEC mask: one issued inside
a lane-masked region still writes its destination in every lane.  A branch
on a value the compiler cannot prove wave-uniform around an MFMA is
compiled to such a region (s_and_saveexec ... s_or_b64 exec) and, unless
the region is skipped with s_cbranch_execz, silently changes the result.
This test compiles every HIP source to assembly and fails on any MFMA in a
masked region that is not skipped.

DPP lane moves have the opposite problem: a lane reading a neighbour that
the mask switched off receives 0 (or its own old value), not the
neighbour's data.  Every lane move in these kernels is written for a full
wave, so the test also fails on any DPP instruction inside a region where
EXEC was narrowed (a select the compiler turned into a branch around a
lane move once cost the backward its cross-row scan).
"""

import os
import re
import subprocess

import pytest

from delta_rule_recurrence_amd import build as B

SOURCES = sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip"))


def _masked_mfmas(asm: str):
    """Linear scan: a saveexec opens a masked region (skipped on an empty mask
    when s_cbranch_execz follows), a restoring s_or_b64 / s_mov_b64 of exec
    closes it.  A saveexec followed by s_cbranch_execnz and an unconditional
    s_branch is a region the block layout placed at the branch target (a
    rotated loop): the text after it is reached only through labels, so it
    leaves the scan's state unchanged."""
    bad, masked, skipped, fn = [], False, False, "?"
    lines = asm.split("\n")

    def nxt(i, k):
        return lines[i + k].strip() if i + k < len(lines) else ""

    for i, line in enumerate(lines):
        if re.match(r"^_Z\S+:", line):
            # a new function starts unmasked
            fn = line.split(":")[0]
            masked, skipped = False, False
        s = line.strip()
        if re.match(r"s_(and|andn2|xor|or)_saveexec", s):
            if nxt(i, 1).startswith("s_cbranch_execnz") and nxt(i, 2).startswith("s_branch"):
                continue
            masked = True
            skipped = nxt(i, 1).startswith("s_cbranch_execz")
        elif s.startswith("s_or_b64 exec") or s.startswith("s_mov_b64 exec"):
            masked = False
        elif s.startswith("v_mfma") and masked and not skipped:
            bad.append(f"{fn} line {i + 1}: {s}")
    return bad


def _masked_dpp(asm: str):
    """DPP instructions between an EXEC-narrowing instruction (a saveexec, or
    a move or AND into exec) and the s_or_b64 that restores it."""
    bad, masked, fn = [], False, "?"
    for i, line in enumerate(asm.split("\n")):
        if re.match(r"^_Z\S+:", line):
            fn = line.split(":")[0]
            masked = False
        s = line.strip()
        if re.match(r"s_(and|andn2|xor|or)_saveexec_b64", s) or s.startswith("s_mov_b64 exec, s") or \
                s.startswith("s_and_b64 exec"):
            masked = True
        elif s.startswith("s_or_b64 exec, exec"):
            masked = False
        elif masked and "_dpp" in s.split(" ")[0]:
            bad.append(f"{fn} line {i + 1}: {s}")
    return bad


def _hipcc():
    try:
        return B.hipcc()
    except RuntimeError:
        return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_mfma_under_exec_mask(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = out.read_text()
    bad = _masked_mfmas(asm)
    assert not bad, "MFMA inside an EXEC-masked region:\n" + "\n".join(bad[:10])
    bad = _masked_dpp(asm)
    assert not bad, "DPP lane move inside an EXEC-narrowed region:\n" + "\n".join(bad[:10])
