"""fconv_act_pool_noalloc (the allocation-free variant of fconv_act_pool, on the library's
static device scratch) against fconv_act_pool, through the C ABI, on calls in a row whose
inputs shrink: the scratch keeps the previous call's contents, and every call must still
match the allocating entry point bit for bit (the same kernels) and the oracle within the
parity tolerance."""
import numpy as np
import pytest

import oracle
import synth
from tests._util import TOL_F32, max_rel_err, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemm_activation_reduction_amd as fc  # noqa: E402


def _case(seed, N, Cin, H, W, Cout, bf16):
    spec = dict(N=N, Cin=Cin, H=H, W=W, Cout=Cout, x_dist=("normal",), w_bound=1.0 / np.sqrt(9 * Cin),
                b_bound=0.1, dtype="bf16" if bf16 else "f32")
    return synth.conv_inputs(spec, seed_cfg=3000 + seed)


def _both(x, w, b, act, pool, bf16):
    N, Cin, H, W = x.shape
    Cout = w.shape[0]
    xd, wd, bd = to_device(x, bf16), to_device(w, bf16), to_device(b)
    shape = (N, Cout) if pool else (N, Cout, H - 2, W - 2)
    code = act | (fc.DT_BF16 if bf16 else fc.DT_F32)
    ref_out = torch.full(shape, float("nan"), dtype=torch.float32, device=xd.device)
    na_out = torch.full(shape, float("nan"), dtype=torch.float32, device=xd.device)
    s = torch.cuda.current_stream()
    fc.fconv_act_pool(xd, wd, bd, N, Cin, H, W, Cout, code, int(pool), ref_out, s)
    fc.fconv_act_pool_noalloc(xd, wd, bd, N, Cin, H, W, Cout, code, int(pool), na_out, s)
    torch.cuda.synchronize()
    return ref_out.cpu().numpy(), na_out.cpu().numpy()


# (seed, N, Cin, H, W, Cout, bf16, act, pool): each call smaller than the one before
CALLS = [
    (1, 8, 16, 120, 100, 64, False, fc.ACT_GELU, 1),      # pooled, 9.6 k partials per image
    (2, 2, 20, 37, 41, 19, False, fc.ACT_MISH2, 1),       # smaller, ragged tiles and channel tails
    (3, 2, 40, 24, 48, 256, True, fc.ACT_GELU, 0),        # bf16 wide kernel, full map
    (4, 1, 3, 9, 16, 8, False, fc.ACT_GELU_TANH, 0),      # smallest: one tile
]


def test_noalloc_matches_allocating_entry_point_on_shrinking_calls():
    for seed, N, Cin, H, W, Cout, bf16, act, pool in CALLS:
        print(f"noalloc call: seed={seed} x=({N},{Cin},{H},{W}) Cout={Cout} bf16={bf16} act={act} pool={pool}",
              flush=True)
        x, w, b = _case(seed, N, Cin, H, W, Cout, bf16)
        ref, got = _both(x, w, b, act, pool, bf16)
        assert np.array_equal(got, ref), seed
        err = max_rel_err(got, oracle.conv_act_pool(x, w, b, act, pool))
        print(f"  bit-equal to fconv_act_pool, oracle err={err:.3e}", flush=True)
        assert err <= TOL_F32
