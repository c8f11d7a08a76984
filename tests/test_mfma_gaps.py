"""Static check of the decode-attention kernels as compiled: every vector ALU
instruction that touches an MFMA's registers -- reads its result, writes its
A/B operands, or writes its C operand where C is not also the result -- comes
at least 8 wait states after that MFMA.

The partition kernels follow each logits MFMA and each P.V pair with a gap
(a scheduling barrier, s_nop 7, a scheduling barrier), because an earlier
build in which a conversion rewrote an MFMA's C registers 3 wait states after
the MFMA gave timing-dependent wrong results.  This test compiles
paged_attention.hip for gfx950 with the library's flags, walks each MFMA's
straight-line successors (up to the next label or branch) counting wait
states (one per instruction, N + 1 for s_nop N), and fails if the compiler
ever places such an instruction closer.  It needs hipcc; it runs no GPU code.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "paged_quantized_kv_amd"))
import build  # noqa: E402  (the library's own compile flags)

MIN_GAP = 8
KERNELS = ("paged_attention_balanced_kernelILi16E", "paged_attention_balanced_kernelILi0E",
           "paged_attention_partition_kernelILi16E", "paged_attention_partition_kernelILi0E")


def _regs(tok):
    """The v/a registers an operand names, as ('v'|'a', index) pairs."""
    tok = tok.strip()
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(ins):
    parts = ins.split(None, 1)
    if len(parts) == 1:
        return parts[0], []
    ops = [o.strip().split()[0] for o in re.split(r",(?![^\[]*\])", parts[1]) if o.strip()]
    return parts[0], ops


def _wait_states(ins):
    op, ops = _operands(ins)
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def kernel_body(asm, name):
    """Instructions of one kernel (labels kept, comments and directives dropped)."""
    lines = asm.splitlines()
    start = next(i for i, l in enumerate(lines) if re.match(rf"^_Z\w*{name}\w*:", l))
    body = []
    for l in lines[start + 1:]:
        s = l.split(";")[0].strip()
        if s.startswith(".LBB"):
            body.append(s)
        elif s and not s.startswith("."):
            body.append(s)
        if s.startswith("s_endpgm"):
            break
    return body


def closest_touches(body, window=120):
    """For each MFMA: (wait states to the nearest VALU instruction that reads
    its result or writes its A, B or C-not-result registers, that MFMA,
    that instruction), for the MFMAs that have one in straight-line code."""
    found = []
    for i, ins in enumerate(body):
        if not ins.startswith("v_mfma"):
            continue
        _, ops = _operands(ins)
        dst, a, b, c = (_regs(o) for o in ops[:4])
        watch_w = a | b | (c - dst if c != dst else set())
        ws = 0
        for nxt in body[i + 1:i + window]:
            if nxt.startswith((".LBB", "s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
                break
            if nxt.startswith("v_") and not nxt.startswith("v_mfma"):
                op, nops = _operands(nxt)
                written = _regs(nops[0]) if nops else set()
                read = set().union(*(_regs(o) for o in nops[1:])) if len(nops) > 1 else set()
                if "_dpp" in op or "fmac" in op or "row_" in nxt or "quad_perm" in nxt:
                    read |= written  # tied or partially written destinations
                if (read & dst) or (written & watch_w):
                    found.append((ws, ins, nxt))
                    break
            ws += _wait_states(nxt)
    return found


def compile_attention_asm(tmp_path):
    hipcc = build.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = tmp_path / "paged_attention.s"
    cmd = [hipcc, *build.CXXFLAGS, "-x", "hip", "-S", "--cuda-device-only",
           os.path.join(build.CSRC, "paged_attention.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_no_valu_touches_an_mfma_within_the_gap(tmp_path):
    asm = compile_attention_asm(tmp_path)
    for name in KERNELS:
        body = kernel_body(asm, name)
        n_mfma = sum(1 for x in body if x.startswith("v_mfma"))
        assert n_mfma >= 48, (name, n_mfma)  # 16 logits + 32 P.V per block at least
        close = [f for f in closest_touches(body) if f[0] < MIN_GAP]
        assert not close, f"{name}: {close[:3]}"


def test_the_scan_catches_a_planted_hazard():
    """A conversion writing an MFMA's C registers 3 wait states after it (the
    pattern of the build that failed), and a read of the result 2 wait states
    after, are both reported; the same code with s_nop 7 in front is not."""
    bad = ["v_mfma_f32_16x16x32_bf16 v[10:13], v[0:3], v[4:7], v[20:23]",
           "v_add_u32_e32 v30, v31, v32",
           "v_mov_b32_e32 v33, v34",
           "v_cvt_pk_bf16_f32 v21, v40, v41",
           "s_endpgm"]
    hits = closest_touches(bad)
    assert len(hits) == 1 and hits[0][0] == 2 and "v21" in hits[0][2]
    raw = ["v_mfma_f32_16x16x32_bf16 v[10:13], v[0:3], v[4:7], v[10:13]",
           "v_mov_b32_e32 v33, v34",
           "v_mul_f32_e32 v35, v11, v36",
           "s_endpgm"]
    hits = closest_touches(raw)
    assert len(hits) == 1 and hits[0][0] == 1
    good = [bad[0], "s_nop 7"] + bad[1:]
    hits = closest_touches(good)
    assert len(hits) == 1 and hits[0][0] >= MIN_GAP
