"""Wait states around the GEMM's inline-assembly MFMAs, checked on the built gfx950 code.

The grouped GEMM issues its MFMAs as inline assembly (the accumulators are pinned to AGPRs that
way), so the compiler's hazard recognizer does not see them and inserts no wait states for them.
Two hazards then have to be excluded by the code itself:
  - a VALU write of a VGPR that an MFMA reads as an operand needs two wait states before the MFMA
    (the compiler's own MFMAs get them; the kernels pin masked or dequantized fragments ahead of
    explicit wait states).  One write is exempt: the compiler masks a scale code it loaded as a
    byte to its low byte in place (v_and 0xff, same register), sometimes right before the MFMA;
    the scaled MFMA reads only that byte of a scale operand, which the mask does not change;
  - an MFMA's result must not be read or overwritten by another instruction before the MFMA is
    done: 18 wait states are asked here, more than the passes of any MFMA the library issues.  The
    compiler may copy accumulators out wherever the kernel's paths join, so this follows the
    control flow: every path from an MFMA to an instruction touching its AGPRs counts.
(A change that let the last K step end on one of two paths gave a copy of an accumulator
one MFMA after it was written, and wrong results in that accumulator's lane.)
The scan is a forward data-flow pass over the basic blocks of the assembly: per AGPR the fewest
wait states since an MFMA wrote it, per VGPR since a VALU wrote it, merged by minimum at joins.
"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_scaled_amd", "csrc")
MFMA_WAIT = 18
VALU_WAIT = 2
MEMORY_OPS = ("global_", "buffer_", "ds_", "flat_", "scratch_")


def _regs(tok, kind):
    m = re.match(kind + r"\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(kind + r"(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _split(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip().split()[0] for o in parts[1].split(",") if o.strip()]


def _blocks(asm):
    """Basic blocks [label, instructions]: split at labels and after branches."""
    blocks, cur, label = [], [], None
    for raw in asm.split("\n"):
        line = raw.split(";")[0].strip()
        if not line or (line.startswith(".") and not line.endswith(":")):
            continue
        if line.endswith(":"):
            if cur or label is not None:
                blocks.append((label, cur))
            label, cur = line[:-1], []
            continue
        cur.append(line)
        if line.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
            blocks.append((label, cur))
            label, cur = None, []
    if cur or label is not None:
        blocks.append((label, cur))
    return blocks


def violations(asm):
    blocks = _blocks(asm)
    where = {lab: i for i, (lab, _) in enumerate(blocks) if lab is not None}
    succ = []
    for i, (_, body) in enumerate(blocks):
        s = []
        op = body[-1].split()[0] if body else ""
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = body[-1].split()[1]
            if tgt in where:
                s.append(where[tgt])
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    state = [None] * len(blocks)
    state[0] = ({}, {})
    work, bad = [0], set()
    while work:
        i = work.pop()
        acc, valu = dict(state[i][0]), dict(state[i][1])
        for line in blocks[i][1]:
            op, ops = _split(line)
            wait = int(ops[0]) + 1 if op == "s_nop" else 1
            if op.startswith("v_mfma"):
                srcs = set()
                for t in ops[1:]:
                    srcs |= _regs(t, "v")
                scales = set()
                if op.startswith("v_mfma_scale") and len(ops) >= 6:
                    scales = _regs(ops[4], "v") | _regs(ops[5], "v")
                for v in srcs:
                    w = valu.get(v)
                    if w is not None and w[0] < VALU_WAIT and not (w[1] and v in scales and v not in srcs - scales):
                        bad.add(("VALU write -> MFMA read", line))
                for a in _regs(ops[0], "a"):
                    acc[a] = -1
            elif op.startswith("v_") or op.startswith(MEMORY_OPS):
                touched = set()
                for t in ops:
                    touched |= _regs(t, "a")
                if any(acc.get(a, MFMA_WAIT) < MFMA_WAIT for a in touched):
                    bad.add(("MFMA write -> AGPR access", line))
                if op.startswith("v_") and ops:
                    # a byte mask in place: v_and_b32 vX, 0xff, vX
                    low_byte = op.startswith("v_and_b32") and len(ops) == 3 and ops[1] == "0xff" and ops[0] == ops[2]
                    for v in _regs(ops[0], "v"):
                        valu[v] = (-1, low_byte)
            acc = {a: w + wait for a, w in acc.items() if w + wait < MFMA_WAIT}
            valu = {v: (w + wait, m) for v, (w, m) in valu.items() if w + wait < VALU_WAIT}
        for s in succ[i]:
            if state[s] is None:
                state[s] = (acc, valu)
                work.append(s)
                continue
            na, nv = dict(state[s][0]), dict(state[s][1])
            changed = False
            for r, w in acc.items():
                if w < na.get(r, 1 << 30):
                    na[r] = w
                    changed = True
            for r, (w, m) in valu.items():
                ow, om = nv.get(r, (1 << 30, True))
                if w < ow or (w == ow and om and not m):
                    nv[r] = (min(w, ow), om and m)
                    changed = True
            if changed:
                state[s] = (na, nv)
                work.append(s)
    return sorted(bad)


def test_scanner_finds_both_hazards():
    valu = ("\tv_and_b32_e32 v1, 0xff, v3\n"
            "\tv_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[8:15], v[16:23], a[0:3], v1, v2 op_sel_hi:[0,0,0]\n"
            "\ts_endpgm\n")
    assert [k for k, _ in violations(valu)] == ["VALU write -> MFMA read"]
    assert violations(valu.replace("\tv_mfma", "\ts_nop 1\n\tv_mfma")) == []
    # the in-place byte mask of a scale operand is exempt, but not of a data operand
    assert violations(valu.replace("v_and_b32_e32 v1, 0xff, v3", "v_and_b32_e32 v1, 0xff, v1")) == []
    data = valu.replace("v_and_b32_e32 v1, 0xff, v3", "v_and_b32_e32 v8, 0xff, v8")
    assert [k for k, _ in violations(data)] == ["VALU write -> MFMA read"]
    # the accumulator read sits on the branch target; the drain is only on the fall-through path
    acc = ("\tv_mfma_scale_f32_16x16x128_f8f6f4 a[248:251], v[8:15], v[16:23], a[248:251], v1, v2 op_sel_hi:[0,0,0]\n"
           "\ts_cbranch_vccnz .LBB0_2\n"
           "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n"
           ".LBB0_2:\n"
           "\tv_accvgpr_read_b32 v62, a248\n"
           "\ts_endpgm\n")
    assert [k for k, _ in violations(acc)] == ["MFMA write -> AGPR access"]
    assert violations(acc.replace("\ts_cbranch_vccnz .LBB0_2\n", "")) == []


def test_gemm_kernels_keep_mfma_wait_states(tmp_path):
    from moe_grouped_scaled_amd.build import FLAGS, HIPCC
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / "gemm_mx.s"
    flags = [f for f in FLAGS if not f.startswith("-W")]
    subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "gemm_mx.hip"), "-o", str(out)],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
    asm = out.read_text()
    # one scan per kernel function
    kernels = re.findall(r"^(_Z\w+):[^\n]*\n(.*?)^\.Lfunc_end", asm, flags=re.M | re.S)
    names = [n for n, _ in kernels]
    assert any("gemm_mxfp8_256" in n for n in names) and any("gemm_nvfp4_256" in n for n in names), names
    for name, body in kernels:
        bad = violations(body)
        assert not bad, (name, bad[:5])
