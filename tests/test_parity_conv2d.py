"""GPU parity of fconv2d_act_pool (K x K kernel, stride, zero padding) against the fp64
CPU oracle, called through the C ABI.

Small and ragged shapes are compared element by element against the full oracle for
every supported geometry; the full-size geometry workloads are compared on sampled
outputs. Tolerance: max |g - o| / (1 + |o|) <= 1e-4 (fp32 inputs), 2e-2 (bf16 inputs).
"""
import numpy as np
import pytest

import oracle
import synth
from tests._util import TOL_BF16, TOL_BF16_ARITH, TOL_F32, max_rel_err, to_device, workload_conv_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemm_activation_reduction_amd as fc  # noqa: E402

ACTS = [fc.ACT_NONE, fc.ACT_GELU, fc.ACT_MISH2, fc.ACT_GELU_TANH]

GEOMS = [(1, 1, 0), (1, 2, 0), (3, 1, 1), (3, 2, 1), (3, 2, 0), (3, 1, 2), (5, 1, 2), (5, 2, 2), (5, 1, 0),
         (5, 2, 4), (3, 2, 2), (1, 2, 0)]

SHAPES = [
    (2, 5, 13, 11, 7),     # odd everything
    (1, 17, 9, 40, 65),    # Cin one past an fp32 chunk, Cout one past an oc tile
    (1, 3, 5, 5, 2),       # tiny map
    (2, 33, 20, 37, 16),   # Cin one past a bf16 chunk
    (1, 40, 19, 45, 200),  # bf16 128-channel tiles: a ragged second tile, element-wise halo
    (1, 64, 17, 48, 144),  # bf16 128-channel tiles: 16 channels in the second tile, 16-byte halo runs
    (1, 8, 11, 24, 129),   # 128-channel tiles: one channel in the second tile
]


def rand_case(seed, N, Cin, H, W, Cout, K, bf16=False):
    spec = dict(N=N, Cin=Cin, H=H, W=W, Cout=Cout, K=K, x_dist=("normal",), w_bound=1.0 / np.sqrt(K * K * Cin),
                b_bound=0.1, dtype="bf16" if bf16 else "f32")
    return synth.conv_inputs(spec, seed_cfg=3000 + seed)


def run_conv2d(x, w, b, stride, pad, act, pool, bf16=False):
    xd, wd, bd = to_device(x, bf16), to_device(w, bf16), to_device(b)
    out = fc.conv2d_act_pool(xd, wd, bd, stride=stride, pad=pad, act=act, pool=bool(pool))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("pool", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("geom", GEOMS)
def test_conv2d_small_shapes_full_compare(geom, shape, pool, bf16):
    K, S, P = geom
    N, Cin, H, W, Cout = shape
    if H + 2 * P < K or W + 2 * P < K:
        pytest.skip("padded input smaller than the kernel")
    act = ACTS[(K + S + P + Cin + pool) % 4]
    x, w, b = rand_case(K * 100 + S * 10 + P + Cin, *shape, K, bf16=bf16)
    got = run_conv2d(x, w, b, S, P, act, pool, bf16)
    ref = oracle.conv2d_act_pool(x, w, b, S, P, act, pool)
    err = max_rel_err(got, ref)
    print(f"geom={geom} shape={shape} pool={pool} act={act} bf16={bf16} err={err:.3e}", flush=True)
    assert err <= (TOL_BF16 if bf16 else TOL_F32)
    assert err <= TOL_BF16_ARITH


def test_conv2d_3x3_valid_is_the_fast_path_bit_for_bit():
    x, w, b = rand_case(1, 2, 20, 30, 41, 70, 3)
    xd, wd, bd = to_device(x), to_device(w), to_device(b)
    for pool in (False, True):
        o1 = fc.conv_act_pool(xd, wd, bd, act="gelu", pool=pool)
        o2 = fc.conv2d_act_pool(xd, wd, bd, stride=1, pad=0, act="gelu", pool=pool)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


def test_conv2d_padding_border_closed_form():
    # x = 1, w = 1, b = 0, act none, 3x3, pad 1: corners sum 4 taps, edges 6, inside 9 (x Cin)
    Cin = 24
    x = np.ones((1, Cin, 40, 70), np.float32)
    w = np.ones((3, Cin, 3, 3), np.float32)
    got = run_conv2d(x, w, np.zeros(3, np.float32), 1, 1, fc.ACT_NONE, 0)
    assert got.shape == (1, 3, 40, 70)
    expect = np.full((40, 70), 9.0 * Cin)
    expect[0, :] = expect[-1, :] = expect[:, 0] = expect[:, -1] = 6.0 * Cin
    expect[0, 0] = expect[0, -1] = expect[-1, 0] = expect[-1, -1] = 4.0 * Cin
    for c in range(3):
        np.testing.assert_array_equal(got[0, c], expect)


@pytest.mark.parametrize("name", ["conv5x5_same_gelu_pool_f32", "conv3x3_s2_gelu_pool_bf16"])
def test_conv2d_full_size_pooled_whole_output(name):
    spec = synth.CONV_WORKLOADS[name]
    K, S, P = synth.conv_geometry(spec)
    bf16 = spec["dtype"] == "bf16"
    x, w, b = workload_conv_inputs(name)
    print(f"{name}: running GPU", flush=True)
    got = run_conv2d(x, w, b, S, P, spec["act"], 1, bf16)
    assert got.shape == (spec["N"], spec["Cout"]) and np.all(np.isfinite(got))
    ref = oracle.conv2d_act_pool(x, w, b, S, P, spec["act"], 1)
    err = max_rel_err(got, ref)
    print(f"{name}: all {got.size} outputs, err={err:.3e}", flush=True)
    assert err <= (TOL_BF16 if bf16 else TOL_F32)
    assert err <= TOL_BF16_ARITH


def test_conv2d_full_size_1x1_full_output_whole():
    # every output of the (32, 128, 192, 192) map, one image at a time
    name = "conv1x1_mish2_full_f32"
    spec = synth.CONV_WORKLOADS[name]
    K, S, P = synth.conv_geometry(spec)
    x, w, b = workload_conv_inputs(name)
    xd, wd, bd = to_device(x), to_device(w), to_device(b)
    print(f"{name}: running GPU", flush=True)
    out = fc.conv2d_act_pool(xd, wd, bd, stride=S, pad=P, act="mish2", pool=False)
    torch.cuda.synchronize()
    N, Cout, OH, OW = out.shape
    assert (OH, OW) == synth.conv_out_size(spec)
    worst = 0.0
    for n in range(N):
        ref = oracle.conv2d_act_pool(np.ascontiguousarray(x[n:n + 1]), w, b, S, P, fc.ACT_MISH2, 0)
        err = max_rel_err(out[n:n + 1].cpu().numpy(), ref)
        worst = max(worst, err)
        assert err <= TOL_F32, (n, err)
    print(f"{name}: all {out.numel()} outputs, err={worst:.3e}", flush=True)


# Layers with at most 32 output channels run the general kernel's 32-channel tile: every
# output of full-size 5x5 (pooled) and 1x1 (full map) layers against the oracle.
def test_conv2d_narrow_layer_tile_full_size_whole_output():
    x, w, b = rand_case(70, 64, 16, 112, 112, 16, 5)
    print("narrow 5x5 layer: running GPU", flush=True)
    got = run_conv2d(x, w, b, 1, 2, fc.ACT_GELU, 1, False)
    assert got.shape == (64, 16) and np.all(np.isfinite(got))
    err = max_rel_err(got, oracle.conv2d_act_pool(x, w, b, 1, 2, fc.ACT_GELU, 1))
    print(f"narrow 5x5 layer: all {got.size} outputs, err={err:.3e}", flush=True)
    assert err <= TOL_F32
    x, w, b = rand_case(71, 8, 64, 192, 192, 32, 1)
    print("narrow 1x1 layer: running GPU", flush=True)
    got = run_conv2d(x, w, b, 1, 0, fc.ACT_MISH2, 0, False)
    assert got.shape == (8, 32, 192, 192) and np.all(np.isfinite(got))
    err = max_rel_err(got, oracle.conv2d_act_pool(x, w, b, 1, 0, fc.ACT_MISH2, 0))
    print(f"narrow 1x1 layer: all {got.size} outputs, err={err:.3e}", flush=True)
    assert err <= TOL_F32


# fp32 1x1 stride-1 layers with W % 4 == 0 and a 16-byte aligned x stage by LDS DMA; an x 4
# bytes past a 16-byte boundary takes the element-wise register path. Both accumulate chunk by
# chunk and channel group by channel group from the bias, so the outputs agree bit for bit:
# ragged rows and columns, a 1-channel second oc tile, a channel tail chunk, a larger image,
# and the 16-, 32- and 64-channel tiles of narrower layers.
@pytest.mark.parametrize("shape", [(1, 64, 17, 48, 144), (2, 8, 11, 24, 129), (3, 40, 21, 36, 200),
                                   (8, 64, 64, 64, 128), (1, 16, 11, 36, 7), (2, 40, 13, 28, 20),
                                   (3, 64, 9, 44, 64), (1, 33, 10, 16, 65)])
def test_conv2d_1x1_f32_dma_matches_register_path(shape):
    x, w, b = rand_case(hash(shape) % 967 + 9, *shape, 1)
    xd = to_device(x)
    flat = torch.empty(xd.numel() + 1, dtype=torch.float32, device=xd.device)
    flat[1:] = xd.reshape(-1)
    xu = flat[1:].view(xd.shape)
    assert xd.data_ptr() % 16 == 0 and xu.data_ptr() % 16 != 0
    wd, bd = to_device(w), to_device(b)
    for act, pool in (("mish2", False), ("gelu", True), ("none", False)):
        o_dma = fc.conv2d_act_pool(xd, wd, bd, stride=1, pad=0, act=act, pool=pool)
        o_reg = fc.conv2d_act_pool(xu, wd, bd, stride=1, pad=0, act=act, pool=pool)
        torch.cuda.synchronize()
        assert torch.equal(o_dma, o_reg), (act, pool)


# fp32 stride-1 layers with K = 3 or 5 and W % 4 == 0 stage by LDS DMA as well (a 16-byte
# aligned x); the same layer with x 4 bytes past a 16-byte boundary takes the register path.
# Both accumulate in the same order, so the outputs agree bit for bit: every padding below K
# (the staged window's offset from a 4-pixel run differs for each), 16-, 32- and 64-channel
# tiles, a 65-channel layer (two oc tiles), channel tails and several chunks.
DMA_KXK = [
    (3, 1, (2, 5, 13, 20, 7)),
    (3, 2, (1, 17, 11, 36, 33)),
    (5, 2, (2, 16, 19, 28, 64)),
    (5, 1, (1, 40, 9, 44, 65)),
    (5, 3, (1, 3, 21, 24, 16)),
    (5, 4, (2, 33, 8, 12, 20)),
    (5, 0, (1, 64, 30, 40, 64)),
    (5, 4, (1, 3, 1, 4, 5)),       # one input row, one 4-pixel run: padding on every side
    (3, 2, (2, 1, 2, 4, 3)),       # one input channel, a 2 x 4 image
]


@pytest.mark.parametrize("K,P,shape", DMA_KXK)
def test_conv2d_kxk_f32_dma_matches_register_path(K, P, shape):
    x, w, b = rand_case(K * 10 + P + hash(shape) % 953, *shape, K)
    xd = to_device(x)
    flat = torch.empty(xd.numel() + 1, dtype=torch.float32, device=xd.device)
    flat[1:] = xd.reshape(-1)
    xu = flat[1:].view(xd.shape)
    assert xd.data_ptr() % 16 == 0 and xu.data_ptr() % 16 != 0
    wd, bd = to_device(w), to_device(b)
    for act, pool in (("gelu", True), ("mish2", False)):
        o_dma = fc.conv2d_act_pool(xd, wd, bd, stride=1, pad=P, act=act, pool=pool)
        o_reg = fc.conv2d_act_pool(xu, wd, bd, stride=1, pad=P, act=act, pool=pool)
        torch.cuda.synchronize()
        assert torch.equal(o_dma, o_reg), (act, pool)
    got = o_dma.cpu().numpy()
    err = max_rel_err(got, oracle.conv2d_act_pool(x, w, b, 1, P, fc.ACT_MISH2, 0))
    print(f"K={K} P={P} shape={shape} err={err:.3e}", flush=True)
    assert err <= TOL_F32


# bf16 "same" 3x3 layers (stride 1, pad 1) of 256 or more output channels with W % 8 == 0
# and a 16-byte aligned x run the wide 3x3 kernel with one pixel of zero padding; an x 2 bytes
# past a 16-byte boundary takes the general kernel. Both accumulate chunk by chunk and tap by
# tap from the bias, so full maps agree bit for bit. Pooled outputs sum per-tile partials of
# different tile shapes (4 or 8 rows), so there both are held to the oracle instead.
SAME_WIDE = [
    (1, 40, 14, 48, 300),   # two chunks (an 8-channel tail), two oc tiles
    (2, 33, 8, 8, 256),     # the narrowest image (one 8-pixel group), a 1-channel tail chunk
    (1, 64, 9, 32, 257),    # exactly one tile column, a 1-channel second oc tile
    (1, 3, 5, 40, 256),     # three input channels, a ragged second tile column
    (3, 96, 13, 24, 256),   # three chunks, three images
    (1, 32, 1, 16, 256),    # a single input row: padding above and below
]


@pytest.mark.parametrize("shape", SAME_WIDE)
def test_conv2d_same_bf16_wide_kernel(shape):
    x, w, b = rand_case(hash(shape) % 941 + 13, *shape, 3, bf16=True)
    xd = to_device(x, True)
    flat = torch.empty(xd.numel() + 1, dtype=torch.bfloat16, device=xd.device)
    flat[1:] = xd.reshape(-1)
    xu = flat[1:].view(xd.shape)
    assert xd.data_ptr() % 16 == 0 and xu.data_ptr() % 16 != 0
    wd, bd = to_device(w, True), to_device(b)
    for k, pool in enumerate((False, True)):
        act = ACTS[(k + hash(shape)) % 4]
        # the library's per-kernel timers name the kernel each call ran
        fc.fconv_profile(True)
        o_wide = fc.conv2d_act_pool(xd, wd, bd, stride=1, pad=1, act=act, pool=pool)
        torch.cuda.synchronize()
        ran_wide = fc.fconv_profile_read("conv3x3_wide_bf16")[1]
        fc.fconv_profile(True)
        o_gen = fc.conv2d_act_pool(xu, wd, bd, stride=1, pad=1, act=act, pool=pool)
        torch.cuda.synchronize()
        ran_gen = fc.fconv_profile_read("conv_general_fused")[1]
        fc.fconv_profile(False)
        assert ran_wide == 1 and ran_gen == 1, (ran_wide, ran_gen)
        if not pool:
            assert torch.equal(o_wide, o_gen), act
        ref = oracle.conv2d_act_pool(x, w, b, 1, 1, act, int(pool))
        err = max_rel_err(o_wide.cpu().numpy(), ref)
        err_gen = max_rel_err(o_gen.cpu().numpy(), ref)
        print(f"same wide shape={shape} act={act} pool={pool} err={err:.3e} (general {err_gen:.3e})", flush=True)
        # bf16 products are exact in fp32 and accumulate in fp32: the fp32 bound applies
        assert err <= TOL_F32 and err_gen <= TOL_F32


def test_conv2d_same_bf16_wide_full_size_pooled():
    # the 16 x 128 x 128^2 -> 256 layer with "same" padding (the bench workload's inputs):
    # every pooled output
    x, w, b = workload_conv_inputs("conv3x3_same_gelu_pool_bf16")
    print("same wide full size: running GPU", flush=True)
    got = run_conv2d(x, w, b, 1, 1, fc.ACT_GELU, 1, True)
    assert got.shape == (16, 256) and np.all(np.isfinite(got))
    err = max_rel_err(got, oracle.conv2d_act_pool(x, w, b, 1, 1, fc.ACT_GELU, 1))
    print(f"same wide full size: all {got.size} outputs, err={err:.3e}", flush=True)
    assert err <= TOL_F32


def _random_case(rng):
    K = int(rng.choice([1, 3, 5]))
    S = int(rng.choice([1, 2]))
    P = int(rng.integers(0, K))
    N = int(rng.integers(1, 3))
    Cin = int(rng.integers(1, 70))
    Cout = int(rng.choice([int(rng.integers(1, 70)), int(rng.integers(120, 300))]))
    H = int(rng.integers(max(1, K - 2 * P), 40))
    W = int(rng.choice([int(rng.integers(max(1, K - 2 * P), 70)), 8 * int(rng.integers(1, 9))]))
    W = max(W, K - 2 * P)
    return K, S, P, N, Cin, H, W, Cout, bool(rng.integers(0, 2)), int(rng.integers(0, 4)), int(rng.integers(0, 2))


@pytest.mark.parametrize("seed", range(64))
def test_conv2d_random_shapes(seed):
    # seeded random geometry, sizes, dtype, activation and pool mode: sizes cross the tile,
    # chunk and channel-tile boundaries at random, and W is often a multiple of 8 so the
    # 16-byte halo paths run as well as the element-wise ones
    rng = np.random.default_rng(7000 + seed)
    K, S, P, N, Cin, H, W, Cout, bf16, act, pool = _random_case(rng)
    print(f"seed={seed} K={K} S={S} P={P} x=({N},{Cin},{H},{W}) Cout={Cout} bf16={bf16} act={act} pool={pool}",
          flush=True)
    x, w, b = rand_case(100 + seed, N, Cin, H, W, Cout, K, bf16=bf16)
    got = run_conv2d(x, w, b, S, P, ACTS[act], pool, bf16)
    ref = oracle.conv2d_act_pool(x, w, b, S, P, ACTS[act], pool)
    err = max_rel_err(got, ref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= (TOL_BF16 if bf16 else TOL_F32)
    assert err <= TOL_BF16_ARITH
