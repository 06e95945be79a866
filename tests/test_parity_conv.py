"""GPU parity of fconv_act_pool against the fp64 CPU oracle (called through the C ABI).

Small and ragged shapes, and every output of the full-size workloads (in the launch
configuration the benchmark times; the full (32, 128, 190, 190) map one image at a
time), are compared element by element against the oracle. Tolerance:
max |g - o| / (1 + |o|) <= 1e-4 for fp32 inputs and 2e-2 for bf16 inputs. The bf16
cases are also held to 1e-4: both sides read the same bf16 bytes, the products are
exact in fp32 and accumulate in fp32, so only fp32 summation and epilogue rounding
separate them, far below 1e-4 at these sizes.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._util import TOL_BF16, TOL_BF16_ARITH, TOL_F32, max_rel_err, to_device, workload_conv_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemm_activation_reduction_amd as fc  # noqa: E402


def run_conv(x, w, b, act, pool, bf16=False, stream=None):
    xd, wd, bd = to_device(x, bf16), to_device(w, bf16), to_device(b)
    out = fc.conv_act_pool(xd, wd, bd, act=act, pool=bool(pool), stream=stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def rand_case(seed, N, Cin, H, W, Cout, bf16=False):
    spec = dict(N=N, Cin=Cin, H=H, W=W, Cout=Cout, x_dist=("normal",), w_bound=1.0 / np.sqrt(9 * Cin),
                b_bound=0.1, dtype="bf16" if bf16 else "f32")
    return synth.conv_inputs(spec, seed_cfg=1000 + seed)


SHAPES = [
    (2, 3, 16, 16, 8),     # the tiny workload's shape
    (3, 5, 37, 37, 19),    # odd everything: ragged tiles, channel and oc tails
    (1, 1, 3, 3, 1),       # smallest valid input
    (2, 17, 11, 40, 65),   # Cin one past a chunk, Cout one past an oc tile, OW % 4 == 2
    (1, 16, 36, 34, 64),   # OW = 32: exactly one tile column, OW % 4 == 0
    (1, 7, 3, 70, 5),      # a single output row
    (2, 33, 20, 21, 16),   # Cin one past a bf16 chunk, odd OW
    # fp32 with W % 4 == 0 stages by LDS DMA: its edges
    (2, 5, 19, 20, 7),     # W a multiple of 4 but not 8, ragged rows and columns
    (1, 16, 11, 36, 33),   # OW = 34: a second tile column holding two pixels
    (3, 1, 3, 12, 64),     # a single output row, one input channel
    (1, 40, 13, 28, 20),   # three chunks, the last holding 8 channels
    (2, 64, 9, 44, 96),    # four full chunks, a second oc tile of 32 channels
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("act", [fc.ACT_NONE, fc.ACT_GELU, fc.ACT_MISH2, fc.ACT_GELU_TANH])
@pytest.mark.parametrize("pool", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
def test_conv_small_shapes_full_compare(shape, pool, act, bf16):
    x, w, b = rand_case(hash(shape) % 997, *shape, bf16=bf16)
    got = run_conv(x, w, b, act, pool, bf16)
    ref = oracle.conv_act_pool(x, w, b, act, pool)
    err = max_rel_err(got, ref)
    print(f"shape={shape} pool={pool} act={act} bf16={bf16} err={err:.3e}", flush=True)
    assert err <= (TOL_BF16 if bf16 else TOL_F32)
    assert err <= TOL_BF16_ARITH


def test_conv_tiny_workload():
    x, w, b = workload_conv_inputs("conv_tiny")
    got = run_conv(x, w, b, fc.ACT_GELU, 1)
    ref = oracle.conv_act_pool(x, w, b, fc.ACT_GELU, 1)
    assert got.shape == (2, 8)
    assert max_rel_err(got, ref) <= TOL_F32


def test_conv_shifted_delta_kernels_exact():
    # w[oc, ic, kh, kw] = [oc == ic][kh == a][kw == c], b = 0, act none -> a shifted copy of x
    N, C, H, W = 2, 20, 21, 35
    x = synth.normal(4242, N * C * H * W).reshape(N, C, H, W)
    for a in range(3):
        for c in range(3):
            w = np.zeros((C, C, 3, 3), np.float32)
            for k in range(C):
                w[k, k, a, c] = 1.0
            got = run_conv(x, w, np.zeros(C, np.float32), fc.ACT_NONE, 0)
            np.testing.assert_array_equal(got, x[:, :, a:a + H - 2, c:c + W - 2])


def test_conv_zero_weights_and_constant_map():
    N, Cin, H, W, Cout = 2, 16, 30, 30, 32
    b = synth.uniform(77, Cout, -2.0, 2.0)
    x = synth.normal(78, N * Cin * H * W).reshape(N, Cin, H, W)
    w0 = np.zeros((Cout, Cin, 3, 3), np.float32)
    for act in (fc.ACT_GELU, fc.ACT_MISH2, fc.ACT_GELU_TANH):
        expect = np.array([oracle.act(float(v), act) for v in b])
        got = run_conv(x, w0, b, act, 1)
        assert max_rel_err(got, np.broadcast_to(expect, got.shape)) <= TOL_F32
        full = run_conv(x, w0, b, act, 0)
        assert max_rel_err(full, np.broadcast_to(expect[None, :, None, None], full.shape)) <= TOL_F32
    xc = np.full((N, Cin, H, W), 0.5, np.float32)
    w = synth.uniform(79, Cout * Cin * 9, -0.1, 0.1).reshape(Cout, Cin, 3, 3)
    pre = b.astype(np.float64) + 0.5 * w.astype(np.float64).sum(axis=(1, 2, 3))
    for act in (fc.ACT_GELU, fc.ACT_MISH2):
        got = run_conv(xc, w, b, act, 1)
        expect = np.array([oracle.act(float(v), act) for v in pre])
        assert max_rel_err(got, np.broadcast_to(expect, got.shape)) <= TOL_F32


def test_conv_deterministic_and_stream():
    x, w, b = rand_case(5, 4, 16, 60, 60, 64)
    xd, wd, bd = to_device(x), to_device(w), to_device(b)
    o1 = fc.conv_act_pool(xd, wd, bd, act="gelu", pool=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2 = fc.conv_act_pool(xd, wd, bd, act="gelu", pool=True, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    o3 = fc.conv_act_pool(xd, wd, bd, act="gelu", pool=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


@pytest.mark.parametrize("name", ["conv_gelu_pool_f32", "conv_gelu_pool_bf16", "conv_gelu_tanh_pool_bf16"])
def test_conv_full_size_pooled_whole_output(name):
    spec = synth.CONV_WORKLOADS[name]
    bf16 = spec["dtype"] == "bf16"
    x, w, b = workload_conv_inputs(name)
    print(f"{name}: running GPU", flush=True)
    got = run_conv(x, w, b, spec["act"], 1, bf16)
    assert got.shape == (spec["N"], spec["Cout"])
    assert np.all(np.isfinite(got))
    ref = oracle.conv_act_pool(x, w, b, spec["act"], 1)
    err = max_rel_err(got, ref)
    print(f"{name}: all {got.size} outputs, err={err:.3e}", flush=True)
    assert err <= (TOL_BF16 if bf16 else TOL_F32)
    assert err <= TOL_BF16_ARITH


# Layers with at most 16 or 32 output channels run the 16- and 32-channel tiles: every output
# of a full-size layer of each against the oracle.
@pytest.mark.parametrize("Cout,bf16", [(16, False), (32, False), (32, True)])
def test_conv_narrow_layer_tiles_full_size_whole_output(Cout, bf16):
    N, Cin, H, W = (16, 128, 128, 128) if bf16 else (64, 16, 224, 224)
    x, w, b = rand_case(60 + Cout + bf16, N, Cin, H, W, Cout, bf16)
    print(f"narrow layer ({N},{Cin},{H},{W}) -> {Cout} bf16={bf16}: running GPU", flush=True)
    got = run_conv(x, w, b, fc.ACT_GELU, 1, bf16)
    assert got.shape == (N, Cout) and np.all(np.isfinite(got))
    ref = oracle.conv_act_pool(x, w, b, fc.ACT_GELU, 1)
    err = max_rel_err(got, ref)
    print(f"narrow layer -> {Cout}: all {got.size} outputs, err={err:.3e}", flush=True)
    assert err <= TOL_BF16_ARITH


def test_conv_full_size_mish2_full_output_whole():
    # every one of the 147.9 M outputs of the (32, 128, 190, 190) map, one image at a time
    name = "conv_mish2_full_f32"
    x, w, b = workload_conv_inputs(name)
    xd, wd, bd = to_device(x), to_device(w), to_device(b)
    print(f"{name}: running GPU", flush=True)
    out = fc.conv_act_pool(xd, wd, bd, act="mish2", pool=False)
    torch.cuda.synchronize()
    N, Cout, OH, OW = out.shape
    assert (N, Cout, OH, OW) == (32, 128, 190, 190)
    worst = 0.0
    for n in range(N):
        ref = oracle.conv_act_pool(np.ascontiguousarray(x[n:n + 1]), w, b, fc.ACT_MISH2, 0)
        err = max_rel_err(out[n:n + 1].cpu().numpy(), ref)
        worst = max(worst, err)
        assert err <= TOL_F32, (n, err)
    print(f"{name}: all {out.numel()} outputs, err={worst:.3e}", flush=True)


@pytest.mark.parametrize("act", ["none", "gelu"])
def test_conv_wide_full_map_repeatable_at_workload_size(act):
    # The 16 x 128 x 128^2 -> 256 bf16 inputs with the full (16, 256, 126, 126) map written:
    # eight launches in a row must agree bit for bit, and every output must match the
    # oracle. A wait that let a wave pass a barrier before its last DMA had landed made
    # about half of such launches wrong in one 16-channel block of one wave.
    name = "conv_gelu_pool_bf16"
    spec = synth.CONV_WORKLOADS[name]
    x, w, b = workload_conv_inputs(name)
    xd, wd, bd = to_device(x, True), to_device(w, True), to_device(b)
    code = {"none": fc.ACT_NONE, "gelu": fc.ACT_GELU}[act]
    print(f"{name} full map act={act}: running GPU", flush=True)
    first = fc.conv_act_pool(xd, wd, bd, act=code, pool=False)
    out = torch.empty_like(first)
    s = torch.cuda.current_stream()
    same = 0
    for _ in range(8):
        out.fill_(float("nan"))
        fc.conv_act_pool(xd, wd, bd, act=code, pool=False, out=out, stream=s)
        same += int(torch.equal(out, first))
    torch.cuda.synchronize()
    ref = oracle.conv_act_pool(x, w, b, code, 0)
    err = max_rel_err(first.cpu().numpy(), ref)
    print(f"{name} full map act={act}: {same} of 8 repeats bit-equal, all {first.numel()} outputs "
          f"err={err:.3e}", flush=True)
    assert same == 8
    assert err <= TOL_F32


def test_conv_pool_repeated_calls_with_changing_shapes():
    # Calls share the library's cached workspace (repacked weights, pool partials), which
    # grows on demand; every call must be right whatever shape the previous one had.
    cases = [(4, 16, 40, 36, 64), (2, 3, 17, 19, 8), (6, 20, 12, 70, 40), (4, 16, 40, 36, 64)]
    for k, shape in enumerate(cases * 2):
        bf16 = k % 3 == 1
        x, w, b = rand_case(50 + k % len(cases), *shape, bf16=bf16)
        got = run_conv(x, w, b, fc.ACT_GELU, 1, bf16)
        ref = oracle.conv_act_pool(x, w, b, fc.ACT_GELU, 1)
        err = max_rel_err(got, ref)
        assert err <= (TOL_BF16 if bf16 else TOL_F32) and err <= TOL_BF16_ARITH, (k, shape, err)


def test_conv_image_near_the_32bit_offset_limit():
    # One image of x is 16 x 10000 x 3300 float32 = 2.112e9 bytes, just under the 2 GiB
    # per-image bound the staging loads' 32-bit byte offsets allow (the library rejects
    # larger images with FCONV_EUNSUPPORTED). The input repeats a seeded base of 2^24
    # normals; outputs are checked at random points and along the last rows and columns,
    # whose halo loads use the largest offsets.
    N, Cin, H, W, Cout = 1, 16, 10000, 3300, 8
    assert Cin * H * W * 4 < 0x7FFF0000
    base = synth.normal(synth.seed_for(40, 0), 1 << 24)
    x = np.resize(base, (N, Cin, H, W))
    w = synth.uniform(synth.seed_for(40, 1), Cout * Cin * 9, -1 / 12, 1 / 12).reshape(Cout, Cin, 3, 3)
    b = synth.uniform(synth.seed_for(40, 2), Cout, -0.1, 0.1)
    xd = to_device(x)
    del x
    print("near-limit image: running GPU", flush=True)
    out = fc.conv_act_pool(xd, to_device(w), to_device(b), act="gelu", pool=False)
    torch.cuda.synchronize()
    OH, OW = H - 2, W - 2
    assert out.shape == (N, Cout, OH, OW) and bool(torch.isfinite(out).all())
    r = np.random.default_rng(41)
    cnt = 20000
    oc, oh, ow = r.integers(0, Cout, cnt), r.integers(0, OH, cnt), r.integers(0, OW, cnt)
    edge_c = np.arange(OW)
    oc = np.concatenate([oc, np.full(OW, Cout - 1), np.full(OH, Cout - 1)])
    oh = np.concatenate([oh, np.full(OW, OH - 1), np.arange(OH)])
    ow = np.concatenate([ow, edge_c, np.full(OH, OW - 1)])
    n = np.zeros_like(oc)
    idx = [torch.from_numpy(a.astype(np.int64)).cuda() for a in (n, oc, oh, ow)]
    got = out[idx[0], idx[1], idx[2], idx[3]].cpu().numpy()
    del out, xd
    ref = oracle.conv_point_sample(np.resize(base, (N, Cin, H, W)), w, b, fc.ACT_GELU, n, oc, oh, ow)
    err = max_rel_err(got, ref)
    print(f"near-limit image: sampled err={err:.3e}", flush=True)
    assert err <= TOL_F32


# bf16 with Cout >= 256 and 16-byte halo loads runs the wide kernel (256 oc per workgroup,
# weights streamed per tap by LDS DMA): one to four chunks with ragged channel tails,
# ragged tile rows and columns, one, two and ragged oc tiles.
WIDE_SHAPES = [
    (1, 32, 10, 40, 256),   # one chunk, exactly one oc tile, 2 x 2 tiles (ragged columns)
    (2, 40, 14, 48, 300),   # two chunks (8-channel tail), two oc tiles (44-channel tail)
    (1, 128, 9, 32, 512),   # four chunks, two full oc tiles, a ragged tile row
    (1, 3, 6, 16, 256),     # a 3-channel chunk, a tile of 4 x 14 outputs
    (1, 96, 34, 64, 256),   # three chunks, 8 tile rows
    (1, 33, 8, 8, 256),     # the narrowest vector-path image (one 8-pixel group), a 1-channel tail chunk
    (3, 65, 11, 24, 257),   # a 1-channel tail chunk, a second oc tile of one channel, 3 images
]


@pytest.mark.parametrize("act", [fc.ACT_NONE, fc.ACT_GELU, fc.ACT_MISH2, fc.ACT_GELU_TANH])
@pytest.mark.parametrize("pool", [0, 1])
@pytest.mark.parametrize("shape", WIDE_SHAPES)
def test_conv_wide_bf16_full_compare(shape, pool, act):
    x, w, b = rand_case(hash(shape) % 991 + 7, *shape, bf16=True)
    got = run_conv(x, w, b, act, pool, True)
    ref = oracle.conv_act_pool(x, w, b, act, pool)
    err = max_rel_err(got, ref)
    print(f"wide shape={shape} pool={pool} act={act} err={err:.3e}", flush=True)
    # bf16 products are exact in fp32 and accumulate in fp32: the fp32 bound applies
    assert err <= TOL_F32


# Grids of more wide workgroups than the device holds at once (two per CU), so slots are
# refilled and the XCD-contiguous tile numbering covers a count that is not a multiple of
# the resident set: 1280 tiles with one 3-channel chunk; 768 tiles with two chunks, two oc
# tiles and ragged tile rows and columns.
WIDE_LARGE_GRID = [
    (40, 3, 66, 66, 256, "gelu", 1),
    (24, 40, 34, 40, 300, "mish2", 0),
    (24, 40, 34, 40, 300, "gelu_tanh", 1),
]


@pytest.mark.parametrize("N,Cin,H,W,Cout,act,pool", WIDE_LARGE_GRID)
def test_conv_wide_large_grid(N, Cin, H, W, Cout, act, pool):
    x, w, b = rand_case(N * 7 + Cin + W, N, Cin, H, W, Cout, bf16=True)
    tiles = N * ((H - 2 + 3) // 4) * ((W - 2 + 31) // 32) * ((Cout + 255) // 256)
    assert tiles > 2 * torch.cuda.get_device_properties(0).multi_processor_count
    xd, wd, bd = to_device(x, True), to_device(w, True), to_device(b)
    got = fc.conv_act_pool(xd, wd, bd, act=act, pool=bool(pool))
    torch.cuda.synchronize()
    ref = oracle.conv_act_pool(x, w, b, {"gelu": fc.ACT_GELU, "mish2": fc.ACT_MISH2,
                                         "gelu_tanh": fc.ACT_GELU_TANH}[act], pool)
    err = max_rel_err(got.cpu().numpy(), ref)
    print(f"wide large grid N={N} Cin={Cin} H={H} W={W} Cout={Cout} act={act} pool={pool} tiles={tiles} "
          f"err={err:.3e}", flush=True)
    assert err <= TOL_F32


@pytest.mark.parametrize("shape", [(2, 40, 14, 48, 300), (1, 96, 34, 64, 256), (24, 40, 34, 40, 300)])
def test_conv_wide_matches_narrow_full_map(shape):
    # An x that starts 2 bytes past a 16-byte boundary takes the narrow kernel's element-wise
    # halo path; both kernels accumulate chunk by chunk and tap by tap from the bias, so the
    # full output maps agree bit for bit.
    x, w, b = rand_case(hash(shape) % 983 + 3, *shape, bf16=True)
    xd = to_device(x, True)
    flat = torch.empty(xd.numel() + 1, dtype=torch.bfloat16, device=xd.device)
    flat[1:] = xd.reshape(-1)
    xu = flat[1:].view(xd.shape)
    assert xd.data_ptr() % 16 == 0 and xu.data_ptr() % 16 != 0
    wd, bd = to_device(w, True), to_device(b)
    fc.fconv_profile(True)
    o_wide = fc.conv_act_pool(xd, wd, bd, act="mish2", pool=False)
    torch.cuda.synchronize()
    ran_wide = fc.fconv_profile_read("conv3x3_wide_bf16")[1]
    fc.fconv_profile(True)
    o_narrow = fc.conv_act_pool(xu, wd, bd, act="mish2", pool=False)
    torch.cuda.synchronize()
    ran_narrow = fc.fconv_profile_read("conv3x3_fused")[1]
    fc.fconv_profile(False)
    assert ran_wide == 1 and ran_narrow == 1, (ran_wide, ran_narrow)  # each call ran the kernel named
    assert torch.equal(o_wide, o_narrow)


# bf16 pooled at the baseline workload's depth (four or more 32-channel chunks) on grids of
# 1024 or more tiles, four or more per CU: ragged channel chunks, tile rows and columns and
# oc tiles; tile counts that do not divide evenly among the CUs or the eight XCDs.
# fp32 layers with W % 4 == 0 and a 16-byte aligned x stage by LDS DMA; an x 4 bytes past a
# 16-byte boundary takes the element-wise register path. Both accumulate chunk by chunk, tap
# by tap and channel group by channel group from the bias, so full maps and pooled outputs
# agree bit for bit: one chunk (16-channel tile), three chunks with an 8-channel tail
# (32-channel tile), four chunks over two oc tiles, and a larger multi-tile image.
@pytest.mark.parametrize("shape", [(2, 5, 19, 20, 7), (1, 40, 13, 28, 20), (2, 64, 9, 44, 96), (4, 64, 66, 68, 128)])
def test_conv_f32_dma_matches_register_path(shape):
    x, w, b = rand_case(hash(shape) % 971 + 5, *shape)
    xd = to_device(x)
    flat = torch.empty(xd.numel() + 1, dtype=torch.float32, device=xd.device)
    flat[1:] = xd.reshape(-1)
    xu = flat[1:].view(xd.shape)
    assert xd.data_ptr() % 16 == 0 and xu.data_ptr() % 16 != 0
    wd, bd = to_device(w), to_device(b)
    for act, pool in (("gelu", True), ("mish2", False), ("gelu_tanh", False)):
        o_dma = fc.conv_act_pool(xd, wd, bd, act=act, pool=pool)
        o_reg = fc.conv_act_pool(xu, wd, bd, act=act, pool=pool)
        torch.cuda.synchronize()
        assert torch.equal(o_dma, o_reg), (act, pool)


WIDE_DEEP_SHAPES = [
    (24, 100, 37, 72, 300),   # 1296 tiles: a 4-channel tail chunk, ragged rows, columns and oc tile
    (75, 128, 30, 40, 256),   # 1050 tiles (not a multiple of 8): exactly four chunks, 7 x 2 tiles per image
    (33, 160, 66, 64, 256),   # 1056 tiles: five chunks (the fifth without an epilogue slice)
]


@pytest.mark.parametrize("act", [fc.ACT_NONE, fc.ACT_GELU, fc.ACT_MISH2, fc.ACT_GELU_TANH])
@pytest.mark.parametrize("shape", WIDE_DEEP_SHAPES)
def test_conv_wide_deep_large_grid_pooled(shape, act):
    N, Cin, H, W, Cout = shape
    tiles = N * ((H - 2 + 3) // 4) * ((W - 2 + 31) // 32) * ((Cout + 255) // 256)
    assert tiles >= 1024 and (Cin + 31) // 32 >= 4
    x, w, b = rand_case(hash(shape) % 977 + 11, *shape, bf16=True)
    print(f"wide deep shape={shape} tiles={tiles} act={act}: running GPU", flush=True)
    got = run_conv(x, w, b, act, 1, True)
    ref = oracle.conv_act_pool(x, w, b, act, 1)
    err = max_rel_err(got, ref)
    print(f"wide deep shape={shape} act={act} err={err:.3e}", flush=True)
    assert err <= TOL_F32
    # run to run: bit-equal
    again = run_conv(x, w, b, act, 1, True)
    assert np.array_equal(got, again)
