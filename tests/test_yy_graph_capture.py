"""HIP graph capture of fconv_act_pool_noalloc, the entry point for callers that cannot
allocate (code under stream capture among them). Its launches are captured once and
replayed four times. Between replays the test does eager work of its own (clearing the
output, switching the input between two images) and synchronizes. Every replay must
equal the eager call on the same input bit for bit: the graph holds the pointers, not the
values, and the kernels write every output and partial they read back, so no replay
depends on memory cleared at capture time."""
import numpy as np
import pytest

import synth
from tests._util import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemm_activation_reduction_amd as fc  # noqa: E402


def _inputs(seed, N, Cin, H, W, Cout, bf16):
    spec = dict(N=N, Cin=Cin, H=H, W=W, Cout=Cout, x_dist=("normal",), w_bound=1.0 / np.sqrt(9 * Cin),
                b_bound=0.1, dtype="bf16" if bf16 else "f32")
    return synth.conv_inputs(spec, seed_cfg=4000 + seed)


# (N, Cin, H, W, Cout, bf16, act, pool): the narrow fp32 kernel with pool partials and the
# bf16 wide kernel writing the full map
CASES = [
    (2, 20, 37, 41, 19, False, fc.ACT_MISH2, 1),
    (2, 40, 24, 48, 256, True, fc.ACT_GELU, 0),
]


@pytest.mark.parametrize("N,Cin,H,W,Cout,bf16,act,pool", CASES)
def test_graph_replays_equal_eager_calls(N, Cin, H, W, Cout, bf16, act, pool):
    print(f"graph capture: x=({N},{Cin},{H},{W}) Cout={Cout} bf16={bf16} act={act} pool={pool}", flush=True)
    x1, w, b = _inputs(1, N, Cin, H, W, Cout, bf16)
    x2, _, _ = _inputs(2, N, Cin, H, W, Cout, bf16)
    x1d, x2d = to_device(x1, bf16), to_device(x2, bf16)
    xd, wd, bd = x1d.clone(), to_device(w, bf16), to_device(b)
    shape = (N, Cout) if pool else (N, Cout, H - 2, W - 2)
    code = act | (fc.DT_BF16 if bf16 else fc.DT_F32)

    def call(out, stream):
        fc.fconv_act_pool_noalloc(xd, wd, bd, N, Cin, H, W, Cout, code, pool, out, stream)

    # eager results for both inputs
    refs = []
    for src in (x1d, x2d):
        xd.copy_(src)
        ref = torch.full(shape, float("nan"), dtype=torch.float32, device=xd.device)
        call(ref, torch.cuda.current_stream())
        torch.cuda.synchronize()
        refs.append(ref)

    # warm-up on a side stream (the library finds its scratch address on a device's first
    # call), then capture one call
    out = torch.full(shape, float("nan"), dtype=torch.float32, device=xd.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out, torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep, k in enumerate((0, 1, 0, 1)):
        out.fill_(float("nan"))
        xd.copy_((x1d, x2d)[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"  replay {rep} on input {k + 1}", flush=True)
        assert torch.equal(out, refs[k]), rep
