"""GPU parity of fgemm_lse_mish and fgemm_lse_mish_bf16 against the fp64 CPU oracle
(called through the C ABI). Tolerance: max |g - o| / (1 + |o|) <= 1e-4.

For bfloat16 operands both sides consume the same bf16 bytes (the oracle widens them
exactly), bf16 x bf16 products are exact in fp32 and accumulate in fp32, so the fp32
bound applies there too; it is far inside the 2e-2 allowed for bf16 inputs."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests._util import TOL_F32, max_rel_err, to_device, workload_gemm_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemm_activation_reduction_amd as fc  # noqa: E402


def run_gemm(X, W, b, scale=4.0, cmin=-10.0, cmax=10.0, stream=None):
    bf16 = X.dtype == np.uint16
    out = fc.gemm_lse_mish(to_device(X, bf16), to_device(W, bf16), to_device(b), scale, cmin, cmax, stream=stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:, 0]


def rand_case(seed, M, K, N, wb=None, dtype="f32"):
    wb = wb if wb is not None else 1.0 / math.sqrt(K)
    return synth.gemm_inputs(dict(M=M, K=K, N=N, w_bound=wb, b_bound=wb, dtype=dtype), seed_cfg=2000 + seed)


# K % 32 == 0 (fp32) / K % 64 == 0 (bf16) with 16-byte aligned operands takes the LDS-DMA
# kernel; (300, 32, 385) is its shortest K (one pair of stages) with ragged rows and columns
# over two tile rows and three tile columns, (513, 96, 400) three tile rows and an odd
# number of stage pairs. (1300, 64, 1000) has 6 x 6 tiles: the first 32 are renumbered per
# XCD and the last 4 are not, and the second group of tile rows is two rows short.
@pytest.mark.parametrize("M,K,N", [(37, 19, 53), (1, 1, 1), (5, 4, 3), (128, 128, 128), (130, 260, 300),
                                   (64, 1000, 129), (257, 33, 1000), (3, 4096, 6144), (300, 32, 385),
                                   (513, 96, 400), (1300, 64, 1000)])
@pytest.mark.parametrize("scale,cmin,cmax", [(4.0, -10.0, 10.0), (4.0, -0.25, 0.5), (-3.0, -1e30, 1e30)])
def test_gemm_small_shapes(M, K, N, scale, cmin, cmax):
    X, W, b = rand_case(M + K + N, M, K, N)
    got = run_gemm(X, W, b, scale, cmin, cmax)
    ref, _ = oracle.gemm_lse_mish(X, W, b, scale, cmin, cmax)
    err = max_rel_err(got, ref)
    print(f"M={M} K={K} N={N} scale={scale} clamp=[{cmin},{cmax}] err={err:.3e}", flush=True)
    assert err <= TOL_F32


@pytest.mark.parametrize("M,K,N", [(37, 19, 53), (1, 1, 1), (5, 8, 3), (128, 128, 128), (130, 264, 300),
                                   (64, 1000, 129), (257, 33, 1000), (3, 4096, 6144), (300, 72, 385),
                                   (300, 64, 385), (513, 192, 400), (1300, 64, 1000)])
@pytest.mark.parametrize("scale,cmin,cmax", [(4.0, -10.0, 10.0), (-3.0, -1e30, 1e30)])
def test_gemm_bf16_small_shapes(M, K, N, scale, cmin, cmax):
    # K % 8 != 0 takes the element-wise load path, K % 8 == 0 the 16-byte one
    X, W, b = rand_case(M + K + N, M, K, N, dtype="bf16")
    got = run_gemm(X, W, b, scale, cmin, cmax)
    ref, _ = oracle.gemm_lse_mish(X, W, b, scale, cmin, cmax)
    err = max_rel_err(got, ref)
    print(f"bf16 M={M} K={K} N={N} scale={scale} clamp=[{cmin},{cmax}] err={err:.3e}", flush=True)
    assert err <= TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemm_unaligned_operands(dtype):
    # operands starting one element past a 16-byte boundary: K would suit the DMA kernel,
    # but the plan must fall back to the element-wise loads
    M, K, N = 70, 128, 200
    X, W, b = rand_case(7, M, K, N, dtype=dtype)
    bf16 = dtype == "bf16"
    def shifted(a):
        d = to_device(np.concatenate([a.reshape(-1)[:1], a.reshape(-1)]), bf16)
        return d[1:].view(a.shape)
    xd, wd = shifted(X), shifted(W)
    assert xd.data_ptr() % 16 != 0 and wd.data_ptr() % 16 != 0
    out = fc.gemm_lse_mish(xd, wd, to_device(b), 4.0, -10.0, 10.0)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_lse_mish(X, W, b, 4.0, -10.0, 10.0)
    err = max_rel_err(out.cpu().numpy()[:, 0], ref)
    print(f"{dtype} unaligned M={M} K={K} N={N} err={err:.3e}", flush=True)
    assert err <= TOL_F32


def test_gemm_constant_rows_closed_form():
    M, K, N = 70, 16, 6144
    X = np.ones((M, K), np.float32)
    W = np.zeros((N, K), np.float32)
    for beta in (0.0, 0.3, 5.0):
        b = np.full(N, beta, np.float32)
        got = run_gemm(X, W, b)
        c = min(max(4.0 * float(np.float32(beta)), -10.0), 10.0)
        z = c + math.log(N)
        expect = z * z * math.tanh(math.log1p(math.exp(z)))
        assert max_rel_err(got, np.full(M, expect)) <= TOL_F32


def test_gemm_all_clamped_magnitude():
    # every value clamps at 10 over 8192 columns: z = 10 + ln 8192 ~ 19, out ~ 361
    M, K, N = 8, 8, 8192
    got = run_gemm(np.ones((M, K), np.float32), np.ones((N, K), np.float32), np.zeros(N, np.float32))
    ref, _ = oracle.gemm_lse_mish(np.ones((M, K), np.float32), np.ones((N, K), np.float32),
                                  np.zeros(N, np.float32), 4.0, -10.0, 10.0)
    assert max_rel_err(got, ref) <= TOL_F32
    assert np.all(np.abs(got - 361.0) < 1.0)


def test_gemm_deterministic_and_stream():
    X, W, b = rand_case(9, 300, 512, 1000)
    xd, wd, bd = to_device(X), to_device(W), to_device(b)
    o1 = fc.gemm_lse_mish(xd, wd, bd)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2 = fc.gemm_lse_mish(xd, wd, bd, stream=s)
    s.synchronize()
    o3 = fc.gemm_lse_mish(xd, wd, bd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


@pytest.mark.parametrize("name", ["gemm_lse_mish_f32", "gemm_lse_mish_bf16"])
def test_gemm_full_size_whole_output(name):
    spec = synth.GEMM_WORKLOADS[name]
    X, W, b = workload_gemm_inputs(name)
    print(f"{name}: running GPU", flush=True)
    got = run_gemm(X, W, b, spec["scale"], spec["cmin"], spec["cmax"])
    assert got.shape == (spec["M"],) and np.all(np.isfinite(got))
    ref, z = oracle.gemm_lse_mish(X, W, b, spec["scale"], spec["cmin"], spec["cmax"])
    err = max_rel_err(got, ref)
    print(f"{name}: all {got.size} rows, err={err:.3e} z range [{z.min():.3f}, {z.max():.3f}]", flush=True)
    assert err <= TOL_F32
    # LSE bounds hold for every row
    lo, hi = spec["cmin"] + math.log(spec["N"]), spec["cmax"] + math.log(spec["N"])
    zz_lo, zz_hi = lo * lo * math.tanh(math.log1p(math.exp(lo))), hi * hi
    assert np.all(got >= min(zz_lo, 0.0) - 1e-3) and np.all(got <= zz_hi + 1e-3)


@pytest.mark.parametrize("dtype,M", [("f32", 140000), ("bf16", 270000)])
def test_gemm_operand_over_2gib(dtype, M):
    # x of more than 2 GiB (but under 2^31 elements): too large for the LDS-DMA kernel's
    # 31-bit buffer offsets, so the plan takes the register-staged kernel, whose row
    # offsets are 64-bit. x repeats a 1024-row random block; rows sampled from the first
    # block, the middle and the far end (byte offsets past 2^31) are checked.
    K, N = 4096, 200
    Xb, W, b = rand_case(11, 1024, K, N, dtype=dtype)
    X = np.tile(Xb, (M // 1024 + 1, 1))[:M]
    esz = 2 if dtype == "bf16" else 4
    assert M * K * esz > 2 ** 31 and M * K < 2 ** 31
    got = run_gemm(X, W, b)
    rows = np.array([0, 1, 1023, M // 2, M - 1025, M - 2, M - 1])
    ref, _ = oracle.gemm_lse_mish(X[rows], W, b, 4.0, -10.0, 10.0)
    err = max_rel_err(got[rows], ref)
    print(f"{dtype} M={M} K={K} N={N} ({M * K * esz / 2 ** 30:.2f} GiB) sampled err={err:.3e}", flush=True)
    assert err <= TOL_F32
    # rows that repeat the same block row give the same result
    assert np.array_equal(got[rows[1:3]], got[rows[1:3] + 1024 * 100])


def test_concurrent_streams_bit_equal():
    # three streams with different work enqueued interleaved (no synchronization between
    # them): each stream has its own library workspace, so every result must equal the one
    # computed alone on the default stream, bit for bit
    import synth as sy
    spec_a = dict(N=3, Cin=16, H=70, W=90, Cout=80, act=1, pool=1, dtype="f32", x_dist=("normal",),
                  w_bound=1 / 12, b_bound=0.1)
    spec_b = dict(N=2, Cin=40, H=40, W=48, Cout=64, act=2, pool=0, dtype="bf16", x_dist=("normal",),
                  w_bound=0.05, b_bound=0.1)
    xa, wa, ba = sy.conv_inputs(spec_a, seed_cfg=801)
    xb, wb, bb = sy.conv_inputs(spec_b, seed_cfg=802)
    X, W, b = rand_case(803, 300, 256, 700)
    da = (to_device(xa), to_device(wa), to_device(ba))
    db = (to_device(xb, True), to_device(wb, True), to_device(bb))
    dg = (to_device(X), to_device(W), to_device(b))
    ref_a = fc.conv_act_pool(*da, act="gelu", pool=True)
    ref_b = fc.conv_act_pool(*db, act="mish2", pool=False)
    ref_g = fc.gemm_lse_mish(*dg, 4.0, -10.0, 10.0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    outs = {0: [], 1: [], 2: []}
    for _ in range(4):
        with torch.cuda.stream(streams[0]):
            outs[0].append(fc.conv_act_pool(*da, act="gelu", pool=True, stream=streams[0]))
        with torch.cuda.stream(streams[1]):
            outs[1].append(fc.conv_act_pool(*db, act="mish2", pool=False, stream=streams[1]))
        with torch.cuda.stream(streams[2]):
            outs[2].append(fc.gemm_lse_mish(*dg, 4.0, -10.0, 10.0, stream=streams[2]))
    torch.cuda.synchronize()
    for o in outs[0]:
        assert torch.equal(o, ref_a)
    for o in outs[1]:
        assert torch.equal(o, ref_b)
    for o in outs[2]:
        assert torch.equal(o, ref_g)


@pytest.mark.parametrize("seed", range(16))
def test_gemm_random_shapes(seed):
    # seeded random sizes (K often a multiple of the 64-byte stage so the LDS-DMA path runs,
    # otherwise the register-staged one), scale and clamp window, either dtype
    rng = np.random.default_rng(8000 + seed)
    dtype = "bf16" if rng.integers(0, 2) else "f32"
    M = int(rng.integers(1, 700))
    N = int(rng.integers(1, 1500))
    stage = 32 if dtype == "bf16" else 16
    K = int(rng.choice([int(rng.integers(1, 400)), stage * 2 * int(rng.integers(1, 12))]))
    scale = float(rng.choice([4.0, -2.5, 0.5]))
    cmin = float(rng.uniform(-12.0, 0.0))
    cmax = float(cmin + rng.uniform(0.0, 20.0))
    print(f"seed={seed} {dtype} M={M} K={K} N={N} scale={scale} clamp=[{cmin:.3f},{cmax:.3f}]", flush=True)
    X, W, b = rand_case(500 + seed, M, K, N, dtype=dtype)
    got = run_gemm(X, W, b, scale, cmin, cmax)
    ref, _ = oracle.gemm_lse_mish(X, W, b, scale, cmin, cmax)
    err = max_rel_err(got, ref)
    print(f"  err={err:.3e}", flush=True)
    assert err <= TOL_F32
