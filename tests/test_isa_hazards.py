"""Generated-code check for a hazard the compiler cannot guard.

The fused forward and the backward issue their MFMAs through inline asm, to pin
accumulators and operands to AGPRs. The compiler then does not know these
instructions are MFMAs, so its hazard recognizer does not insert the wait states
a VALU write needs before an MFMA reads the written register. Where the kernels
write MFMA operands on the VALU themselves (packed P and dS), they add the wait
states in their own asm. But when register pressure makes the compiler spill an
operand to an AGPR, it can reload it with v_accvgpr_read right in front of the
asm MFMA, and the MFMA then reads a stale register. That gave wrong gradients in
two variants of the dK/dV kernel at d = 64 that were not kept.

This test compiles the kernels to gfx950 assembly and fails if any MFMA reads a
register that a VALU instruction (v_accvgpr_read included) wrote fewer than two
wait states before. CPU only: hipcc cross-compiles without a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_softmax_attn_amd", "csrc")
SOURCES = ["fa_fwd.hip", "fa_bwd.hip"]
MIN_WAIT_STATES = 2


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return path if os.path.exists(path) else None


def _regs(tok):
    m = re.match(r"([av])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _functions(asm_text):
    """name -> list of instruction lines (labels, comments and directives dropped)."""
    out = {}
    for m in re.finditer(r"^(_Z\S*kernel\S*):", asm_text, re.M):
        name = m.group(1)
        end = asm_text.index(".Lfunc_end", m.end())
        lines = [l.strip() for l in asm_text[m.end():end].split("\n")]
        out[name] = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
    return out


def _hazards(instrs):
    """(index, writer, mfma) for MFMAs that read a register a VALU instruction wrote
    fewer than MIN_WAIT_STATES wait states earlier."""
    found = []
    for k, line in enumerate(instrs):
        if not line.startswith("v_mfma"):
            continue
        ops = [t.rstrip(",") for t in line.split()[1:]]
        sources = set().union(*[_regs(t) for t in ops[1:]])
        waits = 0
        for back in range(1, 6):
            if k - back < 0 or waits >= MIN_WAIT_STATES:
                break
            prev = instrs[k - back]
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1]) + 1
                continue
            if prev.startswith("v_") and not prev.startswith("v_mfma"):
                fields = prev.split()
                written = _regs(fields[1].rstrip(",")) if len(fields) > 1 else set()
                if written & sources:
                    found.append((k, prev, line))
                    break
            waits += 1
    return found


def test_hazard_scan_finds_a_planted_case():
    """The scanner itself: a reload right in front of an MFMA is found, and two wait
    states (or an unrelated register) clear it."""
    bad = ["v_accvgpr_read_b32 v91, a107", "v_mfma_f32_32x32x16_bf16 v[16:31], v[88:91], a[72:75], v[16:31]"]
    ok_nop = ["v_accvgpr_read_b32 v91, a107", "s_nop 1",
              "v_mfma_f32_32x32x16_bf16 v[16:31], v[88:91], a[72:75], v[16:31]"]
    ok_other = ["v_accvgpr_read_b32 v95, a107", "v_mfma_f32_32x32x16_bf16 v[16:31], v[88:91], a[72:75], v[16:31]"]
    assert len(_hazards(bad)) == 1
    assert _hazards(ok_nop) == [] and _hazards(ok_other) == []


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_valu_write_feeds_an_mfma_without_wait_states(tmp_path, src):
    out = str(tmp_path / (src + ".s"))
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-w", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        funcs = _functions(f.read())
    assert funcs, "no kernels found in the generated assembly"
    problems = {name: _hazards(body) for name, body in funcs.items()}
    problems = {k: v for k, v in problems.items() if v}
    assert not problems, "\n".join(f"{k}: {v[:3]}" for k, v in problems.items())
