"""Shared helpers for the parity tests: error metric, input caching, device transfer."""
import functools

import numpy as np

import synth

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# bf16 inputs: both sides read the same bf16 bytes, products are exact in fp32 and
# accumulate in fp32, so the fp32 bound also holds (2e-2 stays the acceptance bar)
TOL_BF16_ARITH = 1e-4


def max_rel_err(got, ref) -> float:
    """max |g - o| / (1 + |o|): allclose(atol = rtol = tol) in one number (the pages'
    fp32 convention is atol = rtol = 1e-4)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))


@functools.lru_cache(maxsize=4)
def workload_conv_inputs(name: str):
    return synth.conv_inputs(synth.CONV_WORKLOADS[name])


@functools.lru_cache(maxsize=2)
def workload_gemm_inputs(name: str):
    return synth.gemm_inputs(synth.GEMM_WORKLOADS[name])


def to_device(a: np.ndarray, bf16: bool = False):
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()
