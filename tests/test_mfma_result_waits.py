"""The attention kernels are compiled with their MFMA accumulators in VGPRs
(-amdgpu-mfma-vgpr-form).  An MFMA's result may be read or overwritten only
some wait states after it issues (more for more passes), and the compiler
inserts them: in this build it keeps at least 9 issue slots after each
16x16x32 bf16 product and 11 after each 8-pass fp32 one.  A whole-tile branch
placed between a score product and its first use once left a read 3 slots
behind the MFMA on one path (silently wrong scores on the GPU).  This check
compiles cross_attention.hip to gfx950 assembly with the build's own flags
and fails if, on any path (fall-through and branch targets), a VALU, store or
LDS-write instruction touches an MFMA's destination within 8 issue slots
(each instruction one slot, s_nop n counts n + 1): closer than any distance
the compiler places itself.  It runs on the CPU: hipcc cross-compiles."""

import os
import re
import shutil
import subprocess

import pytest

from block_diffusion_drafter_all_amd import build as BLD

WINDOW = 8
_REG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)\b")


def _vregs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _close_touches(body, window):
    """(MFMA, instruction, slots) for every instruction that touches an MFMA's
    destination VGPRs within ``window`` issue slots of it."""
    labels = {line[:-1]: k for k, line in enumerate(body) if line.endswith(":")}
    found = []
    for k, line in enumerate(body):
        if not line.startswith("v_mfma"):
            continue
        dst = _vregs(line.split(None, 1)[1].split(",")[0])
        stack, seen = [(k + 1, 0)], set()
        while stack:
            m, slots = stack.pop()
            while m < len(body) and slots < window:
                if (m, slots) in seen:
                    break
                seen.add((m, slots))
                ins = body[m]
                m += 1
                if ins.endswith(":"):
                    continue
                if ins.startswith("s_nop"):
                    slots += int(ins.split()[1]) + 1
                    continue
                slots += 1
                if ins.startswith(("s_cbranch", "s_branch")):
                    target = ins.split()[1]
                    if target in labels:
                        stack.append((labels[target], slots))
                    if ins.startswith("s_branch"):
                        break
                    continue
                if ins.startswith("v_mfma"):
                    continue
                if ins.startswith(("v_", "buffer_store", "global_store", "ds_write")):
                    ops = ins.split(None, 1)[1] if " " in ins else ""
                    if _vregs(ops) & dst:
                        found.append((line, ins, slots))
                        break
    return found


def _kernels(asm):
    lines = asm.split("\n")
    starts = [k for k, line in enumerate(lines) if re.match(r"^_Z\S*kernel\S*:", line)]
    for s in starts:
        e = s
        while e < len(lines) and not lines[e].startswith(".Lfunc_end"):
            e += 1
        body = [x.strip() for x in lines[s + 1:e] if x.strip() and not x.strip().startswith(";")]
        yield lines[s].split(":")[0], body


def test_scanner_flags_a_close_read():
    # a read 3 slots behind an MFMA, reached through a branch
    body = ["v_mfma_f32_16x16x32_bf16 v[82:85], v[82:85], v[50:53], v[92:95]",
            "v_mov_b32_e32 v86, 0", "s_cbranch_scc1 .LBB0_9", "v_mov_b32_e32 v1, 0", "s_nop 7", "s_nop 7",
            ".LBB0_9:", "v_fmac_f32_e32 v88, s45, v84"]
    assert [t[2] for t in _close_touches(body, WINDOW)] == [3]
    # the same read 11 slots later on every path passes
    body_ok = body[:2] + ["s_nop 7"] + body[2:]
    assert _close_touches(body_ok, WINDOW) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is not installed")
def test_cross_attention_mfma_results_waited_for(tmp_path):
    src = "cross_attention.hip"
    out = tmp_path / "cross_attention.s"
    cmd = [BLD._hipcc(), *BLD.COMMON_FLAGS, *BLD.SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           os.path.join(BLD.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    bad = {}
    n = 0
    for name, body in _kernels(out.read_text()):
        n += 1
        touches = _close_touches(body, WINDOW)
        if touches:
            bad[name] = touches[:3]
    assert n > 0, "no kernels found in the assembly"
    assert not bad, f"MFMA results touched within {WINDOW} issue slots: {bad}"
