"""Host check of the wide bf16 conv kernel's compiled code (gfx950 assembly built here).

The kernel's main loop waits on the vector-memory counter with hand-counted immediates
(s_waitcnt vmcnt(n)) that count only its LDS DMA instructions (buffer_load ... lds), which
complete in issue order. That is sound only while every vector-memory instruction in the
loop is one of those DMAs: an ordinary load placed among them by the compiler would shift
the count and let a wave pass a barrier before its own DMA had landed. This test compiles
the kernel source and checks, for every instantiation, that the code between the end of
the prologue and the last barrier holds no other vector-memory instruction and no scratch
access.
"""
import os
import re
import shutil
import subprocess

import pytest

from gemm_activation_reduction_amd import build as libbuild

HIPCC = libbuild.HIPCC
SRC = os.path.join(libbuild.CSRC, "conv3x3.hip")
VMEM = re.compile(r"\b(buffer_load|buffer_store|global_load|global_store|flat_load|flat_store|scratch_)")


@pytest.fixture(scope="module")
def wide_asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "conv3x3.s")
    flags = [f for f in libbuild.FLAGS if f != "-fPIC"]
    subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", SRC, "-o", out], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.PIPE)
    lines = open(out).read().split("\n")
    kernels = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S*conv3x3_wide_bf16\S*):", l)
        if m:
            end = next(j for j in range(i, len(lines)) if "s_endpgm" in lines[j])
            kernels[m.group(1)] = lines[i:end]
    return kernels


def test_every_wide_instantiation_found(wide_asm):
    # four activations x pooled / full map
    assert len(wide_asm) == 8


def test_wide_main_loop_vector_memory_is_dma_only(wide_asm):
    for name, body in wide_asm.items():
        bars = [i for i, l in enumerate(body) if "s_barrier" in l]
        # prologue: halo + first DMA steps, barrier, transpose, barrier; the loop follows
        assert len(bars) >= 20, (name, len(bars))
        loop = body[bars[1]:bars[-1]]
        other = [l.strip() for l in loop if VMEM.search(l) and not l.rstrip().endswith(" lds")]
        dma = [l for l in loop if VMEM.search(l) and l.rstrip().endswith(" lds")]
        assert not other, (name, other[:4])
        assert dma, name


def test_wide_kernels_do_not_spill(wide_asm):
    for name, body in wide_asm.items():
        assert not any("scratch_" in l for l in body), name
