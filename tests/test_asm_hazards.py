"""Hazard scan of the attention kernel's inline-asm MFMAs (CPU only).

The score MFMAs of the bf16 attention kernel are written as inline asm, which
the compiler's hazard recognizer does not look into. This test compiles the
kernel source to gfx950 assembly and checks every instantiation:

* before each asm MFMA, no VALU instruction writes one of its source VGPRs
  within the two wait states such a write needs (counting each instruction as
  one wait state and ``s_nop N`` as N + 1);
* after each asm MFMA, no instruction outside the asm chain reads or writes
  its result VGPRs within 18 wait states (the chain's own MFMAs, which take
  the result as their accumulator, are allowed).

A planted hazard (an unguarded MFMA right after a VALU write of its operand)
is checked to be caught, so the scan itself is pinned.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "head_latent_attention_09_amd", "csrc", "mla_attn.hip")
HIPCC = "/opt/rocm/bin/hipcc"
KERNELS = [f"_ZN3mla2mf16attn_mfma_kernelILi{n}ELb{s}ELb{p}EEEvNS0_4ArgsE"
           for n in (1, 2, 3, 4) for s, p in ((0, 0), (1, 0), (1, 1))]
PRE_WAIT = 2      # VALU write of a VGPR -> MFMA read of it
POST_WAIT = 18    # 16x16x32 MFMA result -> any other access


def _vgprs(text: str) -> set[int]:
    out: set[int] = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _instructions(asm: str, kernel: str):
    """(text, in_asm_block) per instruction of one kernel body."""
    body = asm[asm.index(kernel + ":"):]
    body = body[:body.index("s_endpgm")]
    out, in_asm = [], False
    for line in body.split("\n"):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
            continue
        out.append((t.split(";")[0].strip(), in_asm))
    return out


def _waits(text: str) -> int:
    m = re.match(r"s_nop\s+(\d+)", text)
    return int(m.group(1)) + 1 if m else 1


def _operands(text: str):
    op = text.split()[0]
    return op, [x.strip() for x in text[len(op):].split(",")]


def scan(asm: str, kernel: str) -> list[str]:
    ins = _instructions(asm, kernel)
    bad = []
    for i, (text, in_asm) in enumerate(ins):
        if not (in_asm and text.startswith("v_mfma")):
            continue
        _, ops = _operands(text)
        dst = _vgprs(ops[0])
        srcs = set().union(*[_vgprs(x) for x in ops[1:]])
        # backwards: wait states between a VALU write of a source and this MFMA
        w, j = 0, i - 1
        while j >= 0 and w < PRE_WAIT:
            t, a = ins[j]
            if t.startswith("v_") and not t.startswith("v_mfma"):
                _, o = _operands(t)
                if _vgprs(o[0]) & srcs:
                    bad.append(f"{kernel}: VALU write {w} wait states before MFMA: {t} -> {text}")
            w += _waits(t)
            j -= 1
        # forwards: accesses of the result before it is ready
        w, j = 0, i + 1
        while j < len(ins) and w < POST_WAIT:
            t, a = ins[j]
            chained = a and t.startswith("v_mfma")
            if not chained and not t.startswith("s_") and (_vgprs(t) & dst):
                bad.append(f"{kernel}: result accessed {w} wait states after MFMA: {text} -> {t}")
            w += _waits(t)
            j += 1
    return bad


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "mla_attn.s"
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "head_latent_attention_09_amd", "csrc")]
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", *inc, "-S", "--cuda-device-only", "-o", str(out), SRC],
                   check=True, capture_output=True)
    return out.read_text()


@pytest.mark.parametrize("kernel", KERNELS)
def test_no_hazard_around_asm_mfma(kernel_asm, kernel):
    assert kernel + ":" in kernel_asm
    bad = scan(kernel_asm, kernel)
    assert not bad, "\n".join(bad[:10])


def test_scan_catches_planted_hazard():
    asm = "\n".join([
        "k:",
        "\tv_mov_b32_e32 v5, v9",
        ";;#ASMSTART",
        "\tv_mfma_f32_16x16x32_bf16 v[10:13], v[2:5], v[6:9], v[10:13]",
        ";;#ASMEND",
        "\tv_add_f32_e32 v20, v10, v11",
        "\ts_endpgm",
    ])
    bad = scan(asm, "k")
    assert any("VALU write" in b for b in bad)
    assert any("result accessed" in b for b in bad)
    guarded = asm.replace(";;#ASMSTART\n", ";;#ASMSTART\n\ts_nop 1\n").replace(
        "\tv_add_f32_e32", "\ts_nop 7\n\ts_nop 7\n\ts_nop 3\n\tv_add_f32_e32")
    assert scan(guarded, "k") == []
