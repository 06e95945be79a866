"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module only draws numbers; it holds none of the method's arithmetic.
Both sides receive the exact same bytes, so a parity difference can only come
from the computation itself.

Generator: SplitMix64 used counter-style. Draw i of stream ``seed`` is
``mix(seed + (i + 1) * 0x9E3779B97F4A7C15)`` with Steele, Lea and Flood's
finalizer (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014). U[0,1) takes the top 53 bits; N(0,1) uses the
Box-Muller transform on consecutive pairs of uniforms, evaluated in float64 and
rounded to float32 (round-to-nearest-even). bf16 tensors are float32 draws
rounded to bfloat16 with round-to-nearest-even.

Seeds follow ``0x5EED0000 + 16 * config + tensor_id`` (x = 0, w = 1, b = 2).
"""
from __future__ import annotations

import math

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

SEED_BASE = 0x5EED0000
X_ID, W_ID, B_ID = 0, 1, 2


def seed_for(config: int, tensor_id: int) -> int:
    return SEED_BASE + 16 * config + tensor_id


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws ``start .. start+count-1`` of the counter-based SplitMix64 stream."""
    with np.errstate(over="ignore"):
        ctr = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + ctr * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z ^= z >> np.uint64(31)
    return z


def _uniform01(seed: int, start: int, count: int) -> np.ndarray:
    return (splitmix64(seed, start, count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform(seed: int, count: int, lo: float, hi: float) -> np.ndarray:
    """float32 array of U[lo, hi) draws (computed in float64, rounded once)."""
    out = np.empty(count, dtype=np.float32)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        out[s:s + n] = lo + (hi - lo) * _uniform01(seed, s, n)
    return out


def normal(seed: int, count: int) -> np.ndarray:
    """float32 array of N(0, 1) draws by Box-Muller on uniform pairs."""
    out = np.empty(count, dtype=np.float32)
    npairs = (count + 1) // 2
    step = _CHUNK // 2
    for p in range(0, npairs, step):
        n = min(step, npairs - p)
        u = _uniform01(seed, 2 * p, 2 * n)
        r = np.sqrt(-2.0 * np.log1p(-u[0::2]))
        t = (2.0 * math.pi) * u[1::2]
        pair = np.empty(2 * n, dtype=np.float64)
        pair[0::2] = r * np.cos(t)
        pair[1::2] = r * np.sin(t)
        lo = 2 * p
        hi = min(count, lo + 2 * n)
        out[lo:hi] = pair[: hi - lo]
    return out


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Rounds float32 to bfloat16 (round-to-nearest-even); returns uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------
# Workloads. Shapes and distributions are the five configurations the library is
# measured on: a tiny conv, three full-size convs and the GEMM + logsumexp case.
# ----------------------------------------------------------------------------------

ACT_NONE, ACT_GELU, ACT_MISH2, ACT_GELU_TANH = 0, 1, 2, 3

def conv_geometry(spec: dict) -> tuple[int, int, int]:
    """(kernel size, stride, padding) of a conv workload (3, 1, 0 unless stated)."""
    return spec.get("K", 3), spec.get("stride", 1), spec.get("pad", 0)


def conv_out_size(spec: dict) -> tuple[int, int]:
    K, S, P = conv_geometry(spec)
    return (spec["H"] + 2 * P - K) // S + 1, (spec["W"] + 2 * P - K) // S + 1


CONV_WORKLOADS = {
    "conv_tiny": dict(cfg=1, N=2, Cin=3, H=16, W=16, Cout=8, act=ACT_GELU, pool=1, dtype="f32",
                      x_dist=("uniform", -1.0, 1.0), w_bound=1.0 / math.sqrt(27), b_bound=1.0 / math.sqrt(27)),
    "conv_gelu_pool_f32": dict(cfg=2, N=64, Cin=16, H=224, W=224, Cout=64, act=ACT_GELU, pool=1, dtype="f32",
                               x_dist=("normal",), w_bound=1.0 / math.sqrt(16 * 9), b_bound=0.1),
    "conv_mish2_full_f32": dict(cfg=3, N=32, Cin=64, H=192, W=192, Cout=128, act=ACT_MISH2, pool=0, dtype="f32",
                                x_dist=("normal",), w_bound=1.0 / math.sqrt(64 * 9), b_bound=0.1),
    "conv_gelu_pool_bf16": dict(cfg=4, N=16, Cin=128, H=128, W=128, Cout=256, act=ACT_GELU, pool=1, dtype="bf16",
                                x_dist=("normal",), w_bound=1.0 / math.sqrt(128 * 9), b_bound=0.1),
    # general geometry (kernel size K, stride, zero padding): the pages fix K = 3, stride 1,
    # padding 0; these open the three parameters up on the same operator chains
    "conv5x5_same_gelu_pool_f32": dict(cfg=9, N=64, Cin=16, H=224, W=224, Cout=64, K=5, stride=1, pad=2,
                                       act=ACT_GELU, pool=1, dtype="f32", x_dist=("normal",),
                                       w_bound=1.0 / math.sqrt(16 * 25), b_bound=0.1),
    "conv3x3_s2_gelu_pool_bf16": dict(cfg=10, N=16, Cin=128, H=128, W=128, Cout=256, K=3, stride=2, pad=1,
                                      act=ACT_GELU, pool=1, dtype="bf16", x_dist=("normal",),
                                      w_bound=1.0 / math.sqrt(128 * 9), b_bound=0.1),
    "conv1x1_mish2_full_f32": dict(cfg=11, N=32, Cin=64, H=192, W=192, Cout=128, K=1, stride=1, pad=0,
                                   act=ACT_MISH2, pool=0, dtype="f32", x_dist=("normal",),
                                   w_bound=1.0 / math.sqrt(64), b_bound=0.1),
    # the bf16 3x3 layer of the pages' shape with "same" zero padding (output 128 x 128)
    "conv3x3_same_gelu_pool_bf16": dict(cfg=12, N=16, Cin=128, H=128, W=128, Cout=256, K=3, stride=1, pad=1,
                                        act=ACT_GELU, pool=1, dtype="bf16", x_dist=("normal",),
                                        w_bound=1.0 / math.sqrt(128 * 9), b_bound=0.1),
    # the same bf16 inputs (same seeds) with the tanh-approximation GELU epilogue
    "conv_gelu_tanh_pool_bf16": dict(cfg=4, N=16, Cin=128, H=128, W=128, Cout=256, act=ACT_GELU_TANH, pool=1,
                                     dtype="bf16", x_dist=("normal",), w_bound=1.0 / math.sqrt(128 * 9),
                                     b_bound=0.1),
}

GEMM_WORKLOADS = {
    "gemm_lse_mish_f32": dict(cfg=5, M=2048, K=4096, N=6144, scale=4.0, cmin=-10.0, cmax=10.0,
                              w_bound=1.0 / 64, b_bound=1.0 / 64),
    # the same draws (same seeds) with X and W rounded to bfloat16; the bias stays float32
    "gemm_lse_mish_bf16": dict(cfg=5, M=2048, K=4096, N=6144, scale=4.0, cmin=-10.0, cmax=10.0,
                               w_bound=1.0 / 64, b_bound=1.0 / 64, dtype="bf16"),
}


def conv_inputs(spec: dict, seed_cfg: int | None = None):
    """Returns (x, w, b) host arrays for a conv workload spec.

    x: (N, Cin, H, W), w: (Cout, Cin, K, K) (K = spec.get("K", 3)) as float32 or uint16 bf16 bits;
    b: (Cout,) float32.
    ``seed_cfg`` overrides the config number used for seeding (for ad-hoc shapes).
    """
    cfg = spec.get("cfg", 0) if seed_cfg is None else seed_cfg
    N, Cin, H, W, Cout = spec["N"], spec["Cin"], spec["H"], spec["W"], spec["Cout"]
    K = spec.get("K", 3)
    nx, nw = N * Cin * H * W, Cout * Cin * K * K
    dist = spec.get("x_dist", ("normal",))
    if dist[0] == "normal":
        x = normal(seed_for(cfg, X_ID), nx)
    else:
        x = uniform(seed_for(cfg, X_ID), nx, dist[1], dist[2])
    wb, bb = spec["w_bound"], spec["b_bound"]
    w = uniform(seed_for(cfg, W_ID), nw, -wb, wb)
    b = uniform(seed_for(cfg, B_ID), Cout, -bb, bb)
    x = x.reshape(N, Cin, H, W)
    w = w.reshape(Cout, Cin, K, K)
    if spec.get("dtype", "f32") == "bf16":
        x = to_bf16_bits(x).reshape(x.shape)
        w = to_bf16_bits(w).reshape(w.shape)
    return x, w, b


def gemm_inputs(spec: dict, seed_cfg: int | None = None):
    """Returns (X (M,K), W (N,K), b (N,)) host arrays for a GEMM-LSE spec.

    X and W are float32, or uint16 bf16 bits when spec["dtype"] == "bf16"; b is float32.
    """
    cfg = spec.get("cfg", 0) if seed_cfg is None else seed_cfg
    M, K, N = spec["M"], spec["K"], spec["N"]
    X = normal(seed_for(cfg, X_ID), M * K).reshape(M, K)
    W = uniform(seed_for(cfg, W_ID), N * K, -spec["w_bound"], spec["w_bound"]).reshape(N, K)
    b = uniform(seed_for(cfg, B_ID), N, -spec["b_bound"], spec["b_bound"])
    if spec.get("dtype", "f32") == "bf16":
        X = to_bf16_bits(X).reshape(M, K)
        W = to_bf16_bits(W).reshape(N, K)
    return X, W, b


# Epilogue-only workloads: the tensors the pages' own post-conv / post-GEMM kernels read.
# A full-size tensor is a seeded N(0, 1) base of `base` elements repeated to the full
# element count (generating 0.5 G normals on the host would take minutes); every element
# i of the full tensor equals base[i % base].
EPILOGUE_WORKLOADS = {
    # the (128, 64, 254, 254) conv output of the Conv2d(8->64) -> GELU -> avg-pool page
    "epi_gelu_pool_f32": dict(cfg=6, kind="pool", shape=(128, 64, 254, 254), act=ACT_GELU, base=1 << 24),
    # the (64, 128, 254, 254) conv output of the Conv2d(64->128) -> Mish -> Mish page
    "epi_mish2_f32": dict(cfg=7, kind="elementwise", shape=(64, 128, 254, 254), act=ACT_MISH2, base=1 << 24),
    # the (1024, 8192) Linear output of the Linear -> scale -> clamp -> logsumexp -> mish page
    "epi_lse_mish_f32": dict(cfg=8, kind="lse", shape=(1024, 8192), scale=4.0, cmin=-10.0, cmax=10.0,
                             base=1 << 23),
}


def epilogue_base(spec: dict) -> np.ndarray:
    """The seeded float32 N(0, 1) base vector of an epilogue-only workload."""
    total = int(np.prod(spec["shape"]))
    return normal(seed_for(spec["cfg"], X_ID), min(spec["base"], total))


def epilogue_element_indices(spec: dict, flat_index: np.ndarray) -> np.ndarray:
    """Positions in the base vector of the given flat indices of the full tensor."""
    return np.asarray(flat_index, dtype=np.int64) % min(spec["base"], int(np.prod(spec["shape"])))
