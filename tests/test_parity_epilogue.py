"""GPU parity of the epilogue-only entry points (fact_pool, fact_elementwise, flse_mish_rows)
against the fp64 oracle, through the C ABI. Tolerance: max |g - o| / (1 + |o|) <= 1e-4."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests._util import TOL_F32, max_rel_err, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemm_activation_reduction_amd as fc  # noqa: E402

ACTS = [fc.ACT_NONE, fc.ACT_GELU, fc.ACT_MISH2, fc.ACT_GELU_TANH]


def rand(seed, shape, scale=2.0):
    n = int(np.prod(shape))
    return (scale * synth.normal(3000 + seed, n)).astype(np.float32).reshape(shape)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("shape", [(2, 3, 5, 7), (3, 4, 8, 8), (1, 1, 1, 1), (2, 5, 33, 65), (1, 2, 254, 254)])
def test_act_pool_small(shape, act):
    x = rand(sum(shape) + act, shape)
    got = fc.act_pool(to_device(x), act=act)
    torch.cuda.synchronize()
    err = max_rel_err(got.cpu().numpy(), oracle.act_pool_map(x, act))
    print(f"act_pool shape={shape} act={act} err={err:.3e}", flush=True)
    assert err <= TOL_F32


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("count", [1, 3, 4, 5, 1000003])
def test_act_elementwise(count, act):
    x = rand(count + act, (count,), scale=6.0)
    got = fc.act_elementwise(to_device(x), act=act)
    torch.cuda.synchronize()
    assert max_rel_err(got.cpu().numpy(), oracle.act_elementwise(x, act)) <= TOL_F32


def test_act_elementwise_in_place_misaligned_and_empty():
    x = rand(7, (4097,), scale=4.0)
    xd = to_device(x)
    fc.fact_elementwise(xd, x.size, fc.ACT_MISH2, xd)  # in place
    torch.cuda.synchronize()
    assert max_rel_err(xd.cpu().numpy(), oracle.act_elementwise(x, fc.ACT_MISH2)) <= TOL_F32
    # 4-byte (not 16-byte) aligned views take the element path
    xd = to_device(x)
    out = torch.empty(4097, dtype=torch.float32, device="cuda")
    fc.fact_elementwise(xd[1:], 4096, fc.ACT_GELU, out[1:])
    torch.cuda.synchronize()
    assert max_rel_err(out[1:].cpu().numpy(), oracle.act_elementwise(x[1:], fc.ACT_GELU)) <= TOL_F32
    fc.fact_elementwise(xd, 0, fc.ACT_GELU, out)  # count 0 is a no-op


@pytest.mark.parametrize("M,N", [(1, 1), (3, 5), (37, 1000), (16, 8192), (5, 6147)])
# clamp ranges of at most 80 take the one-pass kernel (shift by cmax), wider ones the
# two-pass max-shifted kernel: 80 exactly, just past it, and an unbounded clamp
@pytest.mark.parametrize("scale,cmin,cmax", [(4.0, -10.0, 10.0), (-2.0, -0.5, 3.0), (30.0, -40.0, 40.0),
                                             (30.0, -40.0, 40.5), (3.0, -1e30, 1e30)])
def test_lse_mish_rows(M, N, scale, cmin, cmax):
    y = rand(M * 7 + N, (M, N))
    got = fc.lse_mish_rows(to_device(y), scale, cmin, cmax)
    torch.cuda.synchronize()
    ref, _ = oracle.scale_clamp_lse_mish(y, scale, cmin, cmax)
    err = max_rel_err(got.cpu().numpy()[:, 0], ref)
    print(f"lse_mish_rows M={M} N={N} scale={scale} err={err:.3e}", flush=True)
    assert err <= TOL_F32


def test_lse_mish_rows_all_clamped():
    N = 8192
    y = np.full((4, N), 7.0, np.float32)
    got = fc.lse_mish_rows(to_device(y), 4.0, -10.0, 10.0).cpu().numpy()[:, 0]
    z = 10.0 + math.log(N)
    assert max_rel_err(got, np.full(4, z * z * math.tanh(math.log1p(math.exp(z))))) <= TOL_F32
    # every value at the lower clamp, 80 below the shift: each term is e^-80, still normal in fp32
    y = np.full((4, N), -7.0, np.float32)
    got = fc.lse_mish_rows(to_device(y), 4.0, -40.0, 40.0).cpu().numpy()[:, 0]
    z = -40.0 + math.log(N)
    assert max_rel_err(got, np.full(4, z * z * math.tanh(math.log1p(math.exp(z))))) <= TOL_F32


def test_epilogue_deterministic():
    x = rand(11, (4, 8, 64, 64))
    xd = to_device(x)
    a = fc.act_pool(xd, act="gelu")
    b = fc.act_pool(xd, act="gelu")
    y = to_device(rand(12, (64, 4096)))
    c = fc.lse_mish_rows(y)
    d = fc.lse_mish_rows(y)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


@pytest.mark.parametrize("name", sorted(synth.EPILOGUE_WORKLOADS))
def test_epilogue_workloads_full_size_sampled(name):
    spec = synth.EPILOGUE_WORKLOADS[name]
    base = synth.epilogue_base(spec)
    shape = spec["shape"]
    total = int(np.prod(shape))
    reps = total // base.size
    bd = to_device(base)
    xd = torch.cat([bd.repeat(reps), bd[: total - reps * base.size]]).view(*shape)
    r = np.random.default_rng(9)
    if spec["kind"] == "pool":
        got = fc.act_pool(xd, act=spec["act"]).cpu().numpy()
        N, C, H, W = shape
        planes = r.integers(0, N * C, 24)
        hw = H * W
        ref = np.array([oracle.act_mean(base[synth.epilogue_element_indices(spec, p * hw + np.arange(hw))],
                                        spec["act"]) for p in planes])
        err = max_rel_err(got.reshape(-1)[planes], ref)
    elif spec["kind"] == "elementwise":
        out = fc.act_elementwise(xd, act=spec["act"])
        idx = r.integers(0, total, 200000)
        got = out.view(-1)[torch.from_numpy(idx).cuda()].cpu().numpy()
        ref = oracle.act_elementwise(base[synth.epilogue_element_indices(spec, idx)], spec["act"])
        err = max_rel_err(got, ref)
    else:
        M, N = shape
        got = fc.lse_mish_rows(xd, spec["scale"], spec["cmin"], spec["cmax"]).cpu().numpy()[:, 0]
        rows = r.integers(0, M, 64)
        y = base[synth.epilogue_element_indices(spec, (rows[:, None] * N + np.arange(N)[None, :]).ravel())]
        ref, _ = oracle.scale_clamp_lse_mish(y.reshape(len(rows), N), spec["scale"], spec["cmin"], spec["cmax"])
        err = max_rel_err(got[rows], ref)
    print(f"{name}: sampled err={err:.3e}", flush=True)
    assert err <= TOL_F32
