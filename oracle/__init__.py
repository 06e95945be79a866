"""fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never calls it, and it
never calls the HIP library: the two share no code, only the seeded inputs of
the ``synth`` module.

``oracle.c`` is compiled with gcc (-O2, OpenMP, no fast-math) into
``liboracle.so`` next to this file; :func:`build` does it, and the loader below
refuses to run from a missing library rather than falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants mistakes in a copy of the oracle points this at the copy.
_LIB = os.environ.get("ORACLE_LIB_OVERRIDE", _LIB)

ACT_NONE, ACT_GELU, ACT_MISH2, ACT_GELU_TANH = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compiles oracle.c into liboracle.so (always, when ``force``)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"oracle library missing: {_LIB} (run oracle.build())")
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        lib.oracle_act.argtypes = [ctypes.c_double, ci]
        lib.oracle_act.restype = ctypes.c_double
        for f in ("oracle_gelu", "oracle_gelu_tanh", "oracle_mish", "oracle_softplus"):
            getattr(lib, f).argtypes = [ctypes.c_double]
            getattr(lib, f).restype = ctypes.c_double
        lib.oracle_conv_act_pool.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, dp]
        lib.oracle_conv_pool_sample.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ip, ip, dp]
        lib.oracle_conv_point_sample.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci,
                                                 ip, ip, ip, ip, dp]
        lib.oracle_conv2d_act_pool.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ci, ci, ci, dp]
        lib.oracle_conv2d_pool_sample.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ci, ci,
                                                  ci, ip, ip, dp]
        lib.oracle_conv2d_point_sample.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ci, ci,
                                                   ci, ip, ip, ip, ip, dp]
        lib.oracle_gemm_lse_mish.argtypes = [vp, vp, vp, ci, ci, ci, ci, ctypes.c_double, ctypes.c_double,
                                             ctypes.c_double, ci, ip, dp, dp]
        lib.oracle_lse_mish_rows.argtypes = [dp, ci, ci, dp, dp]
        lib.oracle_num_threads.restype = ci
        lib.oracle_act_mean.argtypes = [vp, ctypes.c_longlong, ci]
        lib.oracle_act_mean.restype = ctypes.c_double
        lib.oracle_act_pool_map.argtypes = [vp, ci, ci, ci, ci, ci, dp]
        lib.oracle_act_elementwise.argtypes = [vp, ctypes.c_longlong, ci, dp]
        lib.oracle_scale_clamp_lse_mish.argtypes = [vp, ci, ci, ctypes.c_double, ctypes.c_double,
                                                    ctypes.c_double, dp, dp]
        _lib = lib
    return _lib


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return 0
    if x.dtype == np.uint16:  # bfloat16 bit patterns
        return 1
    raise TypeError(f"oracle: unsupported input dtype {x.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def act(v: float, kind: int) -> float:
    return _load().oracle_act(float(v), int(kind))


def gelu(v: float) -> float:
    return _load().oracle_gelu(float(v))


def gelu_tanh(v: float) -> float:
    return _load().oracle_gelu_tanh(float(v))


def mish(v: float) -> float:
    return _load().oracle_mish(float(v))


def softplus(v: float) -> float:
    return _load().oracle_softplus(float(v))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _conv_args(x, w, b, K=3):
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    b = np.ascontiguousarray(b, dtype=np.float32)
    code = _dtype_code(x)
    if _dtype_code(w) != code:
        raise TypeError("oracle: x and w must share a dtype")
    N, Cin, H, W = x.shape
    Cout = w.shape[0]
    if w.shape != (Cout, Cin, K, K) or b.shape != (Cout,):
        raise ValueError("oracle: shape mismatch")
    return x, w, b, code, N, Cin, H, W, Cout


def conv_act_pool(x, w, b, act: int, pool: int) -> np.ndarray:
    """Full fused conv in fp64: (N, Cout) if pool else (N, Cout, H-2, W-2)."""
    x, w, b, code, N, Cin, H, W, Cout = _conv_args(x, w, b)
    shape = (N, Cout) if pool else (N, Cout, H - 2, W - 2)
    out = np.empty(shape, dtype=np.float64)
    rc = _load().oracle_conv_act_pool(_ptr(x), _ptr(w), _ptr(b), code, N, Cin, H, W, Cout,
                                      int(act), int(pool), _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_conv_act_pool rc={rc}")
    return out


def conv_pool_sample(x, w, b, act: int, n_idx, oc_idx) -> np.ndarray:
    """Pooled fp64 outputs at the selected (n, oc) pairs."""
    x, w, b, code, N, Cin, H, W, Cout = _conv_args(x, w, b)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int32)
    oc_idx = np.ascontiguousarray(oc_idx, dtype=np.int32)
    out = np.empty(len(n_idx), dtype=np.float64)
    rc = _load().oracle_conv_pool_sample(_ptr(x), _ptr(w), _ptr(b), code, N, Cin, H, W, Cout,
                                         int(act), len(n_idx), _iptr(n_idx), _iptr(oc_idx), _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_conv_pool_sample rc={rc}")
    return out


def conv_point_sample(x, w, b, act: int, n_idx, oc_idx, oh_idx, ow_idx) -> np.ndarray:
    """Activated fp64 outputs at the selected (n, oc, oh, ow) points."""
    x, w, b, code, N, Cin, H, W, Cout = _conv_args(x, w, b)
    idx = [np.ascontiguousarray(a, dtype=np.int32) for a in (n_idx, oc_idx, oh_idx, ow_idx)]
    out = np.empty(len(idx[0]), dtype=np.float64)
    rc = _load().oracle_conv_point_sample(_ptr(x), _ptr(w), _ptr(b), code, N, Cin, H, W, Cout,
                                          int(act), len(idx[0]), *[_iptr(a) for a in idx], _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_conv_point_sample rc={rc}")
    return out


def conv2d_out_size(H: int, W: int, K: int, stride: int, pad: int) -> tuple[int, int]:
    """(OH, OW) of a K x K convolution with the given stride and zero padding."""
    return (H + 2 * pad - K) // stride + 1, (W + 2 * pad - K) // stride + 1


def conv2d_act_pool(x, w, b, stride: int, pad: int, act: int, pool: int) -> np.ndarray:
    """General-geometry fused conv in fp64 (square K x K kernel from w's shape, stride, zero
    padding): (N, Cout) if pool else (N, Cout, OH, OW)."""
    K = int(np.shape(w)[-1])
    x, w, b, code, N, Cin, H, W, Cout = _conv_args(x, w, b, K)
    OH, OW = conv2d_out_size(H, W, K, stride, pad)
    shape = (N, Cout) if pool else (N, Cout, OH, OW)
    out = np.empty(shape, dtype=np.float64)
    rc = _load().oracle_conv2d_act_pool(_ptr(x), _ptr(w), _ptr(b), code, N, Cin, H, W, Cout, K, int(stride),
                                        int(pad), int(act), int(pool), _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_conv2d_act_pool rc={rc}")
    return out


def conv2d_pool_sample(x, w, b, stride: int, pad: int, act: int, n_idx, oc_idx) -> np.ndarray:
    """Pooled fp64 general-geometry outputs at the selected (n, oc) pairs."""
    K = int(np.shape(w)[-1])
    x, w, b, code, N, Cin, H, W, Cout = _conv_args(x, w, b, K)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int32)
    oc_idx = np.ascontiguousarray(oc_idx, dtype=np.int32)
    out = np.empty(len(n_idx), dtype=np.float64)
    rc = _load().oracle_conv2d_pool_sample(_ptr(x), _ptr(w), _ptr(b), code, N, Cin, H, W, Cout, K, int(stride),
                                           int(pad), int(act), len(n_idx), _iptr(n_idx), _iptr(oc_idx),
                                           _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_conv2d_pool_sample rc={rc}")
    return out


def conv2d_point_sample(x, w, b, stride: int, pad: int, act: int, n_idx, oc_idx, oh_idx, ow_idx) -> np.ndarray:
    """Activated fp64 general-geometry outputs at the selected (n, oc, oh, ow) points."""
    K = int(np.shape(w)[-1])
    x, w, b, code, N, Cin, H, W, Cout = _conv_args(x, w, b, K)
    idx = [np.ascontiguousarray(a, dtype=np.int32) for a in (n_idx, oc_idx, oh_idx, ow_idx)]
    out = np.empty(len(idx[0]), dtype=np.float64)
    rc = _load().oracle_conv2d_point_sample(_ptr(x), _ptr(w), _ptr(b), code, N, Cin, H, W, Cout, K, int(stride),
                                            int(pad), int(act), len(idx[0]), *[_iptr(a) for a in idx],
                                            _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_conv2d_point_sample rc={rc}")
    return out


def gemm_lse_mish(X, W, b, scale: float, cmin: float, cmax: float, rows=None):
    """Returns (out, z) in fp64 for all rows, or for the selected ``rows``.

    X and W are both float32, or both uint16 bfloat16 bit patterns (widened exactly)."""
    X = np.ascontiguousarray(X)
    W = np.ascontiguousarray(W)
    b = np.ascontiguousarray(b, dtype=np.float32)
    dt = _dtype_code(X)
    if _dtype_code(W) != dt:
        raise TypeError("oracle: X and W must have the same dtype")
    M, K = X.shape
    N = W.shape[0]
    if W.shape != (N, K) or b.shape != (N,):
        raise ValueError("oracle: shape mismatch")
    if rows is None:
        count, rp, n = 0, None, M
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        count, rp, n = len(rows), _iptr(rows), len(rows)
    out = np.empty(n, dtype=np.float64)
    z = np.empty(n, dtype=np.float64)
    rc = _load().oracle_gemm_lse_mish(_ptr(X), _ptr(W), _ptr(b), dt, M, K, N, float(scale), float(cmin),
                                      float(cmax), count, rp, _dptr(out), _dptr(z))
    if rc != 0:
        raise ValueError(f"oracle_gemm_lse_mish rc={rc}")
    return out, z


def lse_mish_rows(c) -> tuple[np.ndarray, np.ndarray]:
    """logsumexp over each row of an already-clamped fp64 matrix, then z*mish(z)."""
    c = np.ascontiguousarray(c, dtype=np.float64)
    M, N = c.shape
    out = np.empty(M, dtype=np.float64)
    z = np.empty(M, dtype=np.float64)
    rc = _load().oracle_lse_mish_rows(_dptr(c), M, N, _dptr(out), _dptr(z))
    if rc != 0:
        raise ValueError(f"oracle_lse_mish_rows rc={rc}")
    return out, z


# ----------------------------------------------------------------------------- epilogue-only
def act_mean(v, act: int) -> float:
    """Mean of act(v) over a float32 array (one pooled value)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    return float(_load().oracle_act_mean(_ptr(v), v.size, int(act)))


def act_pool_map(x, act: int) -> np.ndarray:
    """(N, C) fp64 means of act(x) over each H x W map of a float32 NCHW array."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, C, H, W = x.shape
    out = np.empty((N, C), dtype=np.float64)
    rc = _load().oracle_act_pool_map(_ptr(x), N, C, H, W, int(act), _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_act_pool_map rc={rc}")
    return out


def act_elementwise(x, act: int) -> np.ndarray:
    """fp64 act(x) elementwise (same shape)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.float64)
    rc = _load().oracle_act_elementwise(_ptr(x), x.size, int(act), _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_act_elementwise rc={rc}")
    return out


def scale_clamp_lse_mish(y, scale: float, cmin: float, cmax: float):
    """(out, z) fp64 per row of a float32 [M][N] matrix: clamp(scale*y) -> logsumexp -> z*mish(z)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    M, N = y.shape
    out = np.empty(M, dtype=np.float64)
    z = np.empty(M, dtype=np.float64)
    rc = _load().oracle_scale_clamp_lse_mish(_ptr(y), M, N, float(scale), float(cmin), float(cmax),
                                             _dptr(out), _dptr(z))
    if rc != 0:
        raise ValueError(f"oracle_scale_clamp_lse_mish rc={rc}")
    return out, z
