"""Python binding of the fconv C ABI (``include/fconv.h``), built as ``libfconv.so``.

Argument marshalling only: every step of the computation runs in the HIP kernels
of the library. PyTorch supplies device memory and the stream. There is no CPU
fallback -- if the library is missing, loading fails loudly.

The functions with the C names (``fconv_act_pool``, ``fgemm_lse_mish``,
``fconv2d_act_pool``, ``fgemm_lse_mish_bf16``, ``fact_pool``, ``fact_elementwise``, ``flse_mish_rows``,
``fconv_last_error``, ``fconv_release``, ``fconv_version``) take the same
arguments as the C entry points; pointer arguments accept a tensor (its
``data_ptr()``) or a plain integer device address, and ``stream`` accepts a
``torch.cuda.Stream``, a raw handle or ``None`` (torch's current stream). A
non-OK status raises :class:`FconvError` carrying the code and the library's
message. ``conv_act_pool`` and ``gemm_lse_mish`` are tensor-level helpers that
allocate the output with torch and call the same entry points.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime first, so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfconv.so")

FCONV_OK, FCONV_EINVAL, FCONV_EUNSUPPORTED, FCONV_EHIP, FCONV_ENOMEM = 0, -1, -2, -3, -4
ACT_NONE, ACT_GELU, ACT_MISH2, ACT_GELU_TANH = 0, 1, 2, 3
DT_F32, DT_BF16 = 0x000, 0x100
_ACT_NAMES = {"none": ACT_NONE, "gelu": ACT_GELU, "mish2": ACT_MISH2, "gelu_tanh": ACT_GELU_TANH}

# Symbols the C header declares; the loader checks that every one is exported.
EXPORTS = ("fconv_act_pool", "fconv_act_pool_noalloc", "fconv2d_act_pool", "fgemm_lse_mish", "fgemm_lse_mish_bf16", "fact_pool", "fact_elementwise", "flse_mish_rows",
           "fconv_last_error", "fconv_release", "fconv_version", "fconv_profile", "fconv_profile_read",
           "fconv_mfma_rate_probe")


class FconvError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"fconv error {code}: {message}")
        self.code = code
        self.message = message


_lib = None


def load_library() -> ctypes.CDLL:
    """Loads libfconv.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with gemm_activation_reduction_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fconv_act_pool.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, vp]
    lib.fconv_act_pool.restype = ci
    lib.fconv_act_pool_noalloc.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, vp]
    lib.fconv_act_pool_noalloc.restype = ci
    lib.fconv2d_act_pool.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ci, ci, vp, vp]
    lib.fconv2d_act_pool.restype = ci
    lib.fgemm_lse_mish.argtypes = [vp, vp, vp, ci, ci, ci, cf, cf, cf, vp, vp]
    lib.fgemm_lse_mish.restype = ci
    lib.fgemm_lse_mish_bf16.argtypes = [vp, vp, vp, ci, ci, ci, cf, cf, cf, vp, vp]
    lib.fgemm_lse_mish_bf16.restype = ci
    lib.fconv_last_error.argtypes = []
    lib.fconv_last_error.restype = ctypes.c_char_p
    lib.fconv_release.argtypes = []
    lib.fconv_release.restype = ci
    lib.fconv_version.argtypes = []
    lib.fconv_version.restype = ci
    lib.fconv_profile.argtypes = [ci]
    lib.fconv_profile.restype = ci
    lib.fconv_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_longlong)]
    lib.fconv_profile_read.restype = ci
    lib.fact_pool.argtypes = [vp, ci, ci, ci, ci, ci, vp, vp]
    lib.fact_pool.restype = ci
    lib.fact_elementwise.argtypes = [vp, ctypes.c_longlong, ci, vp, vp]
    lib.fact_elementwise.restype = ci
    lib.flse_mish_rows.argtypes = [vp, ci, ci, cf, cf, cf, vp, vp]
    lib.flse_mish_rows.restype = ci
    lib.fconv_mfma_rate_probe.argtypes = [ci, ci, vp, ctypes.POINTER(ctypes.c_double), vp]
    lib.fconv_mfma_rate_probe.restype = ci
    for name in EXPORTS:
        getattr(lib, name)
    _lib = lib
    return lib


def _ptr(a) -> int:
    if a is None:
        return 0
    if isinstance(a, torch.Tensor):
        return a.data_ptr()
    return int(a)


def _stream(s) -> int:
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def _check(rc: int) -> None:
    if rc != FCONV_OK:
        raise FconvError(rc, fconv_last_error())


def fconv_last_error() -> str:
    return load_library().fconv_last_error().decode(errors="replace")


def fconv_release() -> None:
    _check(load_library().fconv_release())


def fconv_version() -> int:
    return int(load_library().fconv_version())


def fconv_profile(enable: bool) -> None:
    """Turns per-kernel HIP-event timing on or off (and clears the totals)."""
    _check(load_library().fconv_profile(1 if enable else 0))


def fconv_profile_read(kernel: str) -> tuple[float, int]:
    """(summed event milliseconds, launches) of ``kernel`` since the last fconv_profile()."""
    ms, n = ctypes.c_double(), ctypes.c_longlong()
    _check(load_library().fconv_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def fconv_mfma_rate_probe(dtype, iters, sink, stream=None) -> float:
    """C ``fconv_mfma_rate_probe``: enqueues the MFMA-only rate probe; returns its FLOP count."""
    flops = ctypes.c_double()
    _check(load_library().fconv_mfma_rate_probe(int(dtype), int(iters), _ptr(sink), ctypes.byref(flops),
                                                _stream(stream)))
    return flops.value


def fconv_act_pool(x, w, b, N, Cin, H, W, Cout, act, pool, out, stream=None) -> None:
    """C ``fconv_act_pool``: 3x3 valid conv + bias + activation (+ global mean pool)."""
    rc = load_library().fconv_act_pool(_ptr(x), _ptr(w), _ptr(b), int(N), int(Cin), int(H), int(W), int(Cout),
                                       int(act), int(pool), _ptr(out), _stream(stream))
    _check(rc)


def fconv_act_pool_noalloc(x, w, b, N, Cin, H, W, Cout, act, pool, out, stream=None) -> None:
    """C ``fconv_act_pool_noalloc``: fconv_act_pool on the library's static scratch (no allocation)."""
    rc = load_library().fconv_act_pool_noalloc(_ptr(x), _ptr(w), _ptr(b), int(N), int(Cin), int(H), int(W),
                                               int(Cout), int(act), int(pool), _ptr(out), _stream(stream))
    _check(rc)


def fconv2d_act_pool(x, w, b, N, Cin, H, W, Cout, K, stride, pad, act, pool, out, stream=None) -> None:
    """C ``fconv2d_act_pool``: K x K conv with stride and zero padding + bias + activation (+ mean)."""
    rc = load_library().fconv2d_act_pool(_ptr(x), _ptr(w), _ptr(b), int(N), int(Cin), int(H), int(W), int(Cout),
                                         int(K), int(stride), int(pad), int(act), int(pool), _ptr(out),
                                         _stream(stream))
    _check(rc)


def fgemm_lse_mish(x, w, b, M, K, N, scale, cmin, cmax, out, stream=None) -> None:
    """C ``fgemm_lse_mish``: Linear -> scale -> clamp -> row logsumexp -> z * mish(z)."""
    rc = load_library().fgemm_lse_mish(_ptr(x), _ptr(w), _ptr(b), int(M), int(K), int(N), float(scale),
                                       float(cmin), float(cmax), _ptr(out), _stream(stream))
    _check(rc)


def fgemm_lse_mish_bf16(x, w, b, M, K, N, scale, cmin, cmax, out, stream=None) -> None:
    """C ``fgemm_lse_mish_bf16``: the same chain with bfloat16 x and w (fp32 accumulation)."""
    rc = load_library().fgemm_lse_mish_bf16(_ptr(x), _ptr(w), _ptr(b), int(M), int(K), int(N), float(scale),
                                            float(cmin), float(cmax), _ptr(out), _stream(stream))
    _check(rc)


def fact_pool(x, N, C, H, W, act, out, stream=None) -> None:
    """C ``fact_pool``: act then mean over each (n, c) map of a given float32 NCHW tensor."""
    _check(load_library().fact_pool(_ptr(x), int(N), int(C), int(H), int(W), int(act), _ptr(out), _stream(stream)))


def fact_elementwise(x, count, act, out, stream=None) -> None:
    """C ``fact_elementwise``: out = act(x) elementwise over ``count`` float32 values."""
    _check(load_library().fact_elementwise(_ptr(x), int(count), int(act), _ptr(out), _stream(stream)))


def flse_mish_rows(y, M, N, scale, cmin, cmax, out, stream=None) -> None:
    """C ``flse_mish_rows``: clamp(scale*y) -> row logsumexp -> z*mish(z) over a given [M][N] matrix."""
    _check(load_library().flse_mish_rows(_ptr(y), int(M), int(N), float(scale), float(cmin), float(cmax),
                                         _ptr(out), _stream(stream)))


def _device_of(*tensors) -> torch.device:
    """The one device every tensor sits on (ValueError if they differ)."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"all tensors must be on one device (found {dev} and {t.device})")
    return dev


def _prepare_out(out, shape, device) -> torch.Tensor:
    """A new float32 output of `shape` on `device`, or the caller's `out` once it is checked
    to be a contiguous float32 tensor on `device` with exactly that many elements (any
    shape: the kernels write the elements in that order, every one and nothing beyond)."""
    shape = tuple(int(d) for d in shape)
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    want = 1
    for d in shape:
        want *= d
    if out.dtype != torch.float32 or out.device != device or not out.is_contiguous() or out.numel() != want:
        raise ValueError(f"out must be a contiguous float32 tensor of {want} elements (shape {shape}) on {device}")
    return out


def _act_code(act) -> int:
    return _ACT_NAMES[act] if isinstance(act, str) else int(act)


def conv_act_pool(x: torch.Tensor, w: torch.Tensor, b: torch.Tensor, act="gelu", pool: bool = True,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Tensor helper: x (N,Cin,H,W) and w (Cout,Cin,3,3) float32 or bfloat16, b (Cout,) float32."""
    if x.dtype != w.dtype or x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x and w must both be float32 or both bfloat16")
    if b.dtype != torch.float32:
        raise TypeError("b must be float32")
    for t in (x, w, b):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
    N, Cin, H, W = x.shape
    Cout = w.shape[0]
    if tuple(w.shape) != (Cout, Cin, 3, 3) or tuple(b.shape) != (Cout,):
        raise ValueError("w must be (Cout, Cin, 3, 3) and b (Cout,)")
    dev = _device_of(x, w, b)
    out = _prepare_out(out, (N, Cout) if pool else (N, Cout, H - 2, W - 2), dev)
    code = _act_code(act) | (DT_BF16 if x.dtype == torch.bfloat16 else DT_F32)
    with torch.cuda.device(dev):
        fconv_act_pool(x, w, b, N, Cin, H, W, Cout, code, 1 if pool else 0, out, stream)
    return out


def conv2d_act_pool(x: torch.Tensor, w: torch.Tensor, b: torch.Tensor, stride: int = 1, pad: int = 0, act="gelu",
                    pool: bool = True, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Tensor helper: x (N,Cin,H,W), w (Cout,Cin,K,K) float32 or bfloat16, b (Cout,) float32."""
    if x.dtype != w.dtype or x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x and w must both be float32 or both bfloat16")
    if b.dtype != torch.float32:
        raise TypeError("b must be float32")
    for t in (x, w, b):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
    N, Cin, H, W = x.shape
    Cout, K = w.shape[0], w.shape[-1]
    if tuple(w.shape) != (Cout, Cin, K, K) or tuple(b.shape) != (Cout,):
        raise ValueError("w must be (Cout, Cin, K, K) and b (Cout,)")
    OH, OW = (H + 2 * pad - K) // stride + 1, (W + 2 * pad - K) // stride + 1
    dev = _device_of(x, w, b)
    out = _prepare_out(out, (N, Cout) if pool else (N, Cout, max(OH, 0), max(OW, 0)), dev)
    code = _act_code(act) | (DT_BF16 if x.dtype == torch.bfloat16 else DT_F32)
    with torch.cuda.device(dev):
        fconv2d_act_pool(x, w, b, N, Cin, H, W, Cout, K, stride, pad, code, 1 if pool else 0, out, stream)
    return out


def gemm_lse_mish(x: torch.Tensor, w: torch.Tensor, b: torch.Tensor, scale: float = 4.0, cmin: float = -10.0,
                  cmax: float = 10.0, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Tensor helper: x (M,K), w (N,K) both float32 or both bfloat16, b (N,) float32 -> out (M, 1) float32."""
    if x.dtype != w.dtype or x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x and w must both be float32 or both bfloat16")
    if b.dtype != torch.float32:
        raise TypeError("b must be float32")
    for t in (x, w, b):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
    M, K = x.shape
    N = w.shape[0]
    if tuple(w.shape) != (N, K) or tuple(b.shape) != (N,):
        raise ValueError("w must be (N, K) and b (N,)")
    dev = _device_of(x, w, b)
    out = _prepare_out(out, (M, 1), dev)
    call = fgemm_lse_mish_bf16 if x.dtype == torch.bfloat16 else fgemm_lse_mish
    with torch.cuda.device(dev):
        call(x, w, b, M, K, N, scale, cmin, cmax, out, stream)
    return out


def act_pool(x: torch.Tensor, act="gelu", out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Tensor helper: float32 NCHW x -> (N, C) means of act(x)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 device tensor")
    N, C, H, W = x.shape
    out = _prepare_out(out, (N, C), x.device)
    with torch.cuda.device(x.device):
        fact_pool(x, N, C, H, W, _act_code(act), out, stream)
    return out


def act_elementwise(x: torch.Tensor, act="mish2", out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Tensor helper: float32 x -> act(x) (out may be x itself)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 device tensor")
    out = _prepare_out(out, x.shape, x.device)
    with torch.cuda.device(x.device):
        fact_elementwise(x, x.numel(), _act_code(act), out, stream)
    return out


def lse_mish_rows(y: torch.Tensor, scale: float = 4.0, cmin: float = -10.0, cmax: float = 10.0,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Tensor helper: float32 y (M, N) -> (M, 1)."""
    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous() or y.dim() != 2:
        raise ValueError("y must be a contiguous 2-D float32 device tensor")
    M, N = y.shape
    out = _prepare_out(out, (M, 1), y.device)
    with torch.cuda.device(y.device):
        flse_mish_rows(y, M, N, scale, cmin, cmax, out, stream)
    return out


def loaded_hip_runtimes() -> list[str]:
    """Paths of every libamdhip64 mapped into this process (must be exactly one)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                paths.add(os.path.realpath(parts[-1]))
    return sorted(paths)
