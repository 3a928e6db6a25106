"""The 64-rows-per-wave attention kernels' S^T MFMAs (bf16 and FP8 K/V) are inline asm in
their VGPR form (the compiler would put their accumulators in the AGPRs, which O fills),
so the compiler does not
insert their wait states. This test compiles attn.hip for gfx950 and checks, in the
generated code, the two hazards the asm relies on being absent:
- no vector instruction writes an asm MFMA's A/B/C operands in the 3 instructions
  before it (a vector write must be 2+ wait states ahead of an MFMA read);
- no vector instruction reads an asm MFMA's result registers before the next
  `s_nop` group that the chain's last step carries (the result is not ready).
Needs hipcc; skipped without it."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "..", "block_denoising_step_amd", "csrc", "attn.hip")
# both instantiations (contiguous and paged K/V) of the bf16 and the FP8 kernels
KERNELS = ["_ZN2dg12_GLOBAL__N_122attn_fwd_bf16_d256_w64ILb0EEEvNS0_8AttnArgsE",
           "_ZN2dg12_GLOBAL__N_122attn_fwd_bf16_d256_w64ILb1EEEvNS0_8AttnArgsE",
           "_ZN2dg12_GLOBAL__N_121attn_fwd_fp8_d256_w64ILb0EEEvNS0_8AttnArgsE",
           "_ZN2dg12_GLOBAL__N_121attn_fwd_fp8_d256_w64ILb1EEEvNS0_8AttnArgsE"]


def _regs(op):
    out = set()
    for a, b in re.findall(r"v\[(\d+):(\d+)\]", op):
        out |= set(range(int(a), int(b) + 1))
    for a in re.findall(r"(?<![\[:\w])v(\d+)\b", op):
        out.add(int(a))
    return out


def _asm(tmp_path, kernel):
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc not found")
    out = tmp_path / "attn.s"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-x", "hip", "-S", "--cuda-device-only", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    lines, on = [], False
    for l in out.read_text().splitlines():
        if l.startswith(kernel + ":"):
            on = True
        if on:
            lines.append(l.strip())
            if "s_endpgm" in l:
                break
    assert lines, "kernel not found in the generated code"
    return lines


def _instrs(lines):
    """(index, text, inside asm) for every instruction line."""
    res, in_asm = [], False
    for l in lines:
        if l == ";;#ASMSTART":
            in_asm = True
        elif l == ";;#ASMEND":
            in_asm = False
        elif l and not l.startswith(";") and not l.startswith(".") and not l.endswith(":"):
            res.append((l, in_asm))
    return res


@pytest.mark.parametrize("kernel", KERNELS)
def test_asm_mfma_operands_not_written_just_before(tmp_path, kernel):
    ins = _instrs(_asm(tmp_path, kernel))
    n = 0
    for i, (t, in_asm) in enumerate(ins):
        if not (in_asm and t.startswith("v_mfma")):
            continue
        n += 1
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        srcs = set().union(*(_regs(o) for o in ops[1:]))
        for prev, _ in ins[max(0, i - 3):i]:
            if prev.startswith("v_") and not prev.startswith("v_mfma"):
                assert not (_regs(prev.split(None, 1)[1].split(",")[0]) & srcs), (prev, t)
    assert n >= 32, n  # S^T chains of the loop and the prologue


@pytest.mark.parametrize("kernel", KERNELS)
def test_asm_mfma_results_not_read_before_wait_states(tmp_path, kernel):
    ins = _instrs(_asm(tmp_path, kernel))
    pending = set()  # registers written by asm MFMAs not yet covered by wait states
    for t, in_asm in ins:
        if t.startswith("s_nop 15"):
            pending.clear()
            continue
        if in_asm and t.startswith("v_mfma"):
            ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
            pending |= _regs(ops[0])
            continue
        if t.startswith("v_") or t.startswith("ds_") or t.startswith("global_") or t.startswith("buffer_"):
            parts = t.split(None, 1)
            if len(parts) < 2:
                continue
            ops = [o.strip() for o in parts[1].split(",")]
            reads = set().union(*(_regs(o) for o in (ops[1:] if t.startswith("v_") else ops)))
            if t.startswith("v_mfma") and not in_asm:
                reads = set().union(*(_regs(o) for o in ops[1:]))
            assert not (reads & pending), t
