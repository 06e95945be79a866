"""Run-to-run bit equality of every fused kernel at its full benchmark size.

Each operation is launched six times back to back on one stream, with the output buffer
filled with NaN before every launch, and every result must equal the first bit for bit.
The kernels are atomic-free with a fixed reduction order, so any difference means a
synchronization fault: a wave reading LDS or a partial that another wave or workgroup
has not finished writing. The full sizes matter because such faults depend on how many
workgroups run concurrently and on their timing (one in the wide bf16 convolution showed
only at 16x128x128^2 -> 256 with the full map written).
"""
import pytest

import synth
from tests._util import to_device, workload_conv_inputs, workload_gemm_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemm_activation_reduction_amd as fc  # noqa: E402

REPEATS = 6


def repeat_bit_equal(launch, out):
    first = None
    same = 0
    for _ in range(REPEATS):
        out.fill_(float("nan"))
        launch(out)
        if first is None:
            first = out.clone()
        else:
            same += int(torch.equal(out, first))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(first).all())
    return same


@pytest.mark.parametrize("name", sorted(synth.CONV_WORKLOADS))
@pytest.mark.parametrize("full_map", [False, True])
def test_conv_workloads_repeatable(name, full_map):
    spec = synth.CONV_WORKLOADS[name]
    bf16 = spec["dtype"] == "bf16"
    x, w, b = workload_conv_inputs(name)
    xd, wd, bd = to_device(x, bf16), to_device(w, bf16), to_device(b)
    K, S, P = synth.conv_geometry(spec)
    OH, OW = synth.conv_out_size(spec)
    pool = not full_map
    shape = (spec["N"], spec["Cout"]) if pool else (spec["N"], spec["Cout"], OH, OW)
    out = torch.empty(shape, dtype=torch.float32, device=xd.device)
    if (K, S, P) == (3, 1, 0):
        launch = lambda o: fc.conv_act_pool(xd, wd, bd, act=spec["act"], pool=pool, out=o)
    else:
        launch = lambda o: fc.conv2d_act_pool(xd, wd, bd, stride=S, pad=P, act=spec["act"], pool=pool, out=o)
    print(f"{name} pool={pool}: {REPEATS} launches", flush=True)
    same = repeat_bit_equal(launch, out)
    print(f"{name} pool={pool}: {same} of {REPEATS - 1} repeats bit-equal", flush=True)
    assert same == REPEATS - 1


@pytest.mark.parametrize("name", sorted(synth.GEMM_WORKLOADS))
def test_gemm_workloads_repeatable(name):
    spec = synth.GEMM_WORKLOADS[name]
    bf16 = spec.get("dtype", "f32") == "bf16"
    X, W, b = workload_gemm_inputs(name)
    xd, wd, bd = to_device(X, bf16), to_device(W, bf16), to_device(b)
    out = torch.empty((spec["M"],), dtype=torch.float32, device=xd.device)
    launch = lambda o: fc.gemm_lse_mish(xd, wd, bd, spec["scale"], spec["cmin"], spec["cmax"], out=o)
    print(f"{name}: {REPEATS} launches", flush=True)
    same = repeat_bit_equal(launch, out)
    print(f"{name}: {same} of {REPEATS - 1} repeats bit-equal", flush=True)
    assert same == REPEATS - 1
