"""Static check of the assembly of the kernels with AGPR-pinned accumulators (host only).

The P.V products of `prefill_bf16.hip` and the dV / dK products of `backward.hip` are
MFMAs written as inline assembly, so the
compiler does not know that they keep writing their AGPR accumulators for several cycles
after issue, and it inserts no wait states before a later instruction reads those AGPRs
(a register copy where control flow joins, the epilogue's reads). An early read returns
the value from before the product. This test compiles the file for gfx950 with the
library's own flags and follows every path through each kernel: no `v_accvgpr_read` /
`v_accvgpr_mov` may read an AGPR that such an MFMA wrote fewer than 18 wait states earlier
(a 16-pass XDL op needs at most 18 before a vector read of its result; each instruction
counts one, `s_nop N` counts N + 1).
"""

import os
import re
import shutil
import subprocess

import pytest

from global_attention_qk_amd import build_lib

WAITS = 18


def _agprs(tok):
    m = re.match(r"a\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernels(asm, name):
    lines = asm.split("\n")
    out = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S*" + name + r"\S*):", l)
        if m:
            body = []
            for l2 in lines[i + 1:]:
                s = l2.strip()
                if s.startswith(".Lfunc_end"):   # the kernel's last instruction is above
                    break
                if s and not s.startswith(";") and not s.startswith("."):
                    body.append(s)
                elif re.match(r"^\.LBB\S*:", s):
                    body.append(s)
            out[m.group(1)] = body
    return out


def _early_reads(body):
    """Reads of an AGPR fewer than WAITS wait states after an assembly MFMA wrote it, over
    every path (fall-through and branches, to a fixed point)."""
    labels = {s[:-1]: i for i, s in enumerate(body) if s.endswith(":")}
    # state: AGPR -> wait states since an MFMA wrote it (only those below WAITS)
    entry = [None] * (len(body) + 1)
    entry[0] = {}
    bad = set()
    changed = True
    while changed:
        changed = False
        for i, s in enumerate(body):
            st = entry[i]
            if st is None:
                continue
            st = dict(st)
            op = s.split()[0] if not s.endswith(":") else ""
            if op.startswith(("v_accvgpr_read", "v_accvgpr_mov")):
                for r in _agprs(s.split(",")[1].strip()):
                    if r in st:
                        bad.add((i, s))
            ws = 0 if s.endswith(":") else (int(s.split()[1]) + 1 if op == "s_nop" else 1)
            st = {r: w + ws for r, w in st.items() if w + ws < WAITS}
            if op == "v_mfma_f32_32x32x16_bf16" and " a[" in s:
                for r in _agprs(s.split()[1].rstrip(",")):
                    st[r] = 0
            succ = []
            if op.startswith(("s_cbranch", "s_branch")):
                tgt = s.split()[1]
                if tgt in labels:
                    succ.append(labels[tgt])
            if op not in ("s_branch", "s_endpgm"):   # an early exit ends its path
                succ.append(i + 1)
            for j in succ:
                old = entry[j]
                if old is None:
                    entry[j] = st
                    changed = True
                else:
                    merged = dict(old)
                    for r, w in st.items():
                        if r not in merged or w < merged[r]:
                            merged[r] = w
                    if merged != old:
                        entry[j] = merged
                        changed = True
    return sorted(bad)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src_name,kernel,extra", [
    ("prefill_bf16.hip", "prefill_bf16_kernel", []),
    # the global kernel's other layout (one query block per wave, two waves per SIMD)
    ("prefill_bf16.hip", "prefill_bf16_kernel", ["-DZG_GLOBAL_WAVES=8"]),
    ("backward.hip", "bwd_dkdv_kernel", [])])
def test_no_early_accumulator_reads(tmp_path, src_name, kernel, extra):
    src = os.path.join(build_lib.CSRC, src_name)
    out = tmp_path / (src_name + ".s")
    cmd = [build_lib.hipcc()] + build_lib.common_flags() + extra + [
        "-x", "hip", "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = _kernels(out.read_text(), kernel)
    assert kernels, f"no {kernel} kernels found in the assembly"
    n_mfma = sum(1 for b in kernels.values() for s in b if s.startswith("v_mfma") and " a[" in s)
    assert n_mfma > 0, "no assembly MFMAs with AGPR accumulators found"
    problems = {k: _early_reads(b) for k, b in kernels.items()}
    problems = {k: v for k, v in problems.items() if v}
    assert not problems, {k: v[:3] for k, v in problems.items()}


def test_scanner_flags_an_early_read():
    body = ["v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
            "s_nop 7",
            "v_accvgpr_read_b32 v8, a3"]
    assert _early_reads(body)
    body_ok = ["v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
               "s_nop 7", "s_nop 7", "s_nop 7",
               "v_accvgpr_read_b32 v8, a3"]
    assert not _early_reads(body_ok)
    # through a branch: the read at the target is reached 1 wait state after the MFMA
    body_br = ["s_cbranch_scc1 .LBB0_2",
               "s_nop 7", "s_nop 7", "s_nop 7",
               ".LBB0_1:",
               "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
               "s_cbranch_scc0 .LBB0_2",
               "s_nop 7", "s_nop 7", "s_nop 7",
               ".LBB0_2:",
               "v_accvgpr_mov_b32 a20, a5"]
    assert _early_reads(body_br)
