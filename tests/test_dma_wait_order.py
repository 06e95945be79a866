"""Host check of the compiled code (gfx950 assembly built here) of the two kernels whose
main loops wait with hand-counted vmcnt immediates: the wide bf16 3x3 conv and the
LDS-DMA GEMM-logsumexp.

Their waits (s_waitcnt vmcnt(n) right before a barrier) count only the loop's LDS DMA
instructions (buffer_load ... lds), which complete in issue order. That is sound only
while every vector-memory instruction between the first and the last of those waits is
such a DMA: an ordinary load that the compiler placed (or moved) among them would shift
the count and could let a wave pass a barrier before its own DMA had landed. The test
compiles each source and checks every instantiation.
"""
import os
import re
import shutil
import subprocess

import pytest

from gemm_activation_reduction_amd import build as libbuild

HIPCC = libbuild.HIPCC
VMEM = re.compile(r"\b(buffer_load|buffer_store|global_load|global_store|flat_load|flat_store|scratch_)")
CASES = {"conv3x3.hip": r"conv3x3_wide_bf16", "gemm_lse.hip": r"gemm_lse_partials_dma"}


def compile_kernels(src: str, pattern: str, outdir) -> dict:
    out = str(outdir / (src + ".s"))
    flags = [f for f in libbuild.FLAGS if f != "-fPIC"]
    subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(libbuild.CSRC, src), "-o", out],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
    lines = open(out).read().split("\n")
    kernels = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S*" + pattern + r"\S*):", l)
        if m:
            end = next(j for j in range(i, len(lines)) if "s_endpgm" in lines[j])
            kernels[m.group(1)] = lines[i:end]
    return kernels


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    return {src: compile_kernels(src, pat, d) for src, pat in CASES.items()}


def counted_region(body):
    """Lines from the kernel's first barrier (the end of the prologue) to the last barrier
    preceded by a vmcnt wait (the compiler may schedule a few non-memory instructions, e.g.
    a step's last MFMA, between the two)."""
    code = [l for l in body if l.strip() and not l.strip().startswith(";")]
    bars = [i for i, l in enumerate(code) if "s_barrier" in l]
    marks = [i for i in bars if any("s_waitcnt" in c and "vmcnt" in c for c in code[max(0, i - 4):i])]
    assert len(marks) >= 2
    return code[bars[0]:marks[-1]], len(marks)


def test_instantiations_found(asm):
    assert len(asm["conv3x3.hip"]) == 16         # four activations x pooled / full map x valid / padded
    assert len(asm["gemm_lse.hip"]) == 2         # bf16 and fp32 operands


@pytest.mark.parametrize("src", list(CASES))
def test_counted_region_holds_only_dma(asm, src):
    for name, body in asm[src].items():
        region, waits = counted_region(body)
        other = [l.strip() for l in region if VMEM.search(l) and not l.rstrip().endswith(" lds")]
        dma = [l for l in region if VMEM.search(l)]
        assert not other, (name, other[:4])
        assert dma, name
        assert waits >= 4, (name, waits)


@pytest.mark.parametrize("src", list(CASES))
def test_no_spills(asm, src):
    for name, body in asm[src].items():
        assert not any("scratch_" in l for l in body), name
