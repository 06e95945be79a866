"""C-ABI library checks that need no GPU: every symbol the header declares is exported,
host-side validation rejects bad arguments before any HIP call, only one HIP runtime is
mapped, and the product path never touches the oracle."""
import os
import re
import subprocess

import pytest

import gemm_activation_reduction_amd as fc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fconv.h")
S0 = 0  # explicit null stream: the default (torch's current stream) needs a GPU


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_api():
    assert declared_functions() == sorted(fc.EXPORTS)


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", fc.LIB_PATH], check=True,
                         stdout=subprocess.PIPE).stdout.decode()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in exported, name
    lib = fc.load_library()
    for name in declared_functions():
        assert getattr(lib, name) is not None
    assert fc.fconv_version() == 100


def test_single_hip_runtime_mapped():
    fc.load_library()
    assert len(fc.loaded_hip_runtimes()) == 1, fc.loaded_hip_runtimes()


def test_library_does_not_link_the_oracle():
    out = subprocess.run(["ldd", fc.LIB_PATH], stdout=subprocess.PIPE).stdout.decode()
    assert "oracle" not in out
    pkg = os.path.join(ROOT, "gemm_activation_reduction_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, flags=re.M), f
                assert "liboracle" not in src, f


FAKE = 1 << 40  # plausible, never dereferenced: validation fails before any HIP call


def conv_err(**kw):
    args = dict(x=FAKE, w=FAKE + (1 << 30), b=FAKE + (2 << 30), N=2, Cin=3, H=16, W=16, Cout=8,
                act=fc.ACT_GELU, pool=1, out=FAKE + (3 << 30))
    args.update(kw)
    with pytest.raises(fc.FconvError) as e:
        fc.fconv_act_pool(args["x"], args["w"], args["b"], args["N"], args["Cin"], args["H"], args["W"],
                          args["Cout"], args["act"], args["pool"], args["out"], S0)
    return e.value


@pytest.mark.parametrize("kw,frag", [
    (dict(x=0), "null"), (dict(w=0), "null"), (dict(b=0), "null"), (dict(out=0), "null"),
    (dict(N=0), ">= 1"), (dict(Cin=-1), ">= 1"), (dict(Cout=0), ">= 1"),
    (dict(H=2), ">= 3"), (dict(W=1), ">= 3"),
    (dict(act=4), "unknown activation"), (dict(act=0x200 | 1), "dtype"), (dict(act=0x1000), "dtype"),
    (dict(pool=2), "pool"), (dict(pool=-1), "pool"),
    (dict(N=1 << 16, Cin=1 << 8, H=1 << 8, W=1 << 8), "2^31"),
    (dict(out=FAKE + 64), "overlaps"), (dict(out=FAKE + (1 << 30) + 100), "overlaps"),
])
def test_conv_validation(kw, frag):
    e = conv_err(**kw)
    assert e.code == fc.FCONV_EINVAL
    assert frag in e.message


def gemm_err(**kw):
    args = dict(x=FAKE, w=FAKE + (1 << 30), b=FAKE + (2 << 30), M=4, K=8, N=16, scale=4.0, cmin=-10.0,
                cmax=10.0, out=FAKE + (3 << 30))
    args.update(kw)
    with pytest.raises(fc.FconvError) as e:
        fc.fgemm_lse_mish(args["x"], args["w"], args["b"], args["M"], args["K"], args["N"], args["scale"],
                          args["cmin"], args["cmax"], args["out"], S0)
    return e.value


@pytest.mark.parametrize("kw,frag", [
    (dict(x=0), "null"), (dict(out=0), "null"), (dict(M=0), ">= 1"), (dict(K=-3), ">= 1"), (dict(N=0), ">= 1"),
    (dict(scale=float("inf")), "scale"), (dict(scale=float("nan")), "scale"),
    (dict(cmin=1.0, cmax=-1.0), "cmin"), (dict(cmin=float("nan")), "cmin"),
    (dict(M=1 << 20, K=1 << 12), "2^31"), (dict(out=FAKE + 8), "overlaps"),
])
def test_gemm_validation(kw, frag):
    e = gemm_err(**kw)
    assert e.code == fc.FCONV_EINVAL
    assert frag in e.message


@pytest.mark.parametrize("kw,frag", [
    (dict(w=0), "null"), (dict(M=0), ">= 1"), (dict(scale=float("nan")), "scale"),
    (dict(cmin=2.0, cmax=1.0), "cmin"), (dict(M=1 << 20, K=1 << 12), "2^31"),
    (dict(out=FAKE + 8), "overlaps"),
    # bf16 rows are 2 bytes an element: x covers 4 * 8 * 2 = 64 bytes
    (dict(out=FAKE + 60), "overlaps"),
])
def test_gemm_bf16_validation(kw, frag):
    args = dict(x=FAKE, w=FAKE + (1 << 30), b=FAKE + (2 << 30), M=4, K=8, N=16, scale=4.0, cmin=-10.0,
                cmax=10.0, out=FAKE + (3 << 30))
    args.update(kw)
    with pytest.raises(fc.FconvError) as e:
        fc.fgemm_lse_mish_bf16(args["x"], args["w"], args["b"], args["M"], args["K"], args["N"], args["scale"],
                               args["cmin"], args["cmax"], args["out"], S0)
    assert e.value.code == fc.FCONV_EINVAL
    assert frag in e.value.message
    assert "fgemm_lse_mish_bf16" in e.value.message


def conv2d_err(**kw):
    args = dict(x=FAKE, w=FAKE + (1 << 30), b=FAKE + (2 << 30), N=2, Cin=3, H=16, W=16, Cout=8, K=5, stride=2,
                pad=2, act=fc.ACT_GELU, pool=1, out=FAKE + (3 << 30))
    args.update(kw)
    with pytest.raises(fc.FconvError) as e:
        fc.fconv2d_act_pool(args["x"], args["w"], args["b"], args["N"], args["Cin"], args["H"], args["W"],
                            args["Cout"], args["K"], args["stride"], args["pad"], args["act"], args["pool"],
                            args["out"], S0)
    return e.value


@pytest.mark.parametrize("kw,code,frag", [
    (dict(K=0), fc.FCONV_EINVAL, "K >= 1"), (dict(stride=0), fc.FCONV_EINVAL, "stride >= 1"),
    (dict(pad=-1), fc.FCONV_EINVAL, "pad >= 0"), (dict(H=1, pad=1), fc.FCONV_EINVAL, "smaller than the kernel"),
    (dict(W=2, pad=0), fc.FCONV_EINVAL, "smaller than the kernel"),
    (dict(K=7, pad=3), fc.FCONV_EUNSUPPORTED, "kernel size"), (dict(K=2, pad=0), fc.FCONV_EUNSUPPORTED, "kernel size"),
    (dict(stride=3), fc.FCONV_EUNSUPPORTED, "stride"), (dict(pad=5), fc.FCONV_EUNSUPPORTED, "padding"),
    (dict(act=9), fc.FCONV_EINVAL, "unknown activation"), (dict(x=0), fc.FCONV_EINVAL, "null"),
    (dict(out=FAKE + 64), fc.FCONV_EINVAL, "overlaps"),
    # w is Cout * Cin * K * K = 8 * 3 * 25 float32 = 2400 bytes: out 2396 bytes past w overlaps it
    (dict(out=FAKE + (1 << 30) + 2396), fc.FCONV_EINVAL, "overlaps"),
])
def test_conv2d_validation(kw, code, frag):
    e = conv2d_err(**kw)
    assert e.code == code
    assert frag in e.message
    assert "fconv2d_act_pool" in e.message


def test_last_error_is_per_call():
    conv_err(N=0)
    assert ">= 1" in fc.fconv_last_error()


@pytest.mark.parametrize("call,frag", [
    (lambda: fc.fact_pool(0, 1, 1, 1, 1, 1, FAKE, S0), "null"),
    (lambda: fc.fact_pool(FAKE, 0, 1, 1, 1, 1, FAKE + (1 << 30), S0), ">= 1"),
    (lambda: fc.fact_pool(FAKE, 1, 1, 4, 4, 0x101, FAKE + (1 << 30), S0), "act"),
    (lambda: fc.fact_pool(FAKE, 1, 1, 4, 4, 4, FAKE + (1 << 30), S0), "act"),
    (lambda: fc.fact_pool(FAKE, 1 << 12, 1 << 10, 1 << 5, 1 << 5, 1, FAKE + (1 << 38), S0), "2^31"),
    (lambda: fc.fact_pool(FAKE, 2, 2, 4, 4, 1, FAKE + 16, S0), "overlaps"),
    (lambda: fc.fact_elementwise(FAKE, -1, 1, FAKE + (1 << 30), S0), "count"),
    (lambda: fc.fact_elementwise(FAKE, 100, 7, FAKE + (1 << 30), S0), "act"),
    (lambda: fc.fact_elementwise(FAKE, 100, 1, FAKE + 4, S0), "overlap"),
    (lambda: fc.fact_elementwise(0, 100, 1, FAKE, S0), "null"),
    (lambda: fc.flse_mish_rows(FAKE, 0, 4, 4.0, -1.0, 1.0, FAKE + (1 << 30), S0), ">= 1"),
    (lambda: fc.flse_mish_rows(FAKE, 4, 4, float("inf"), -1.0, 1.0, FAKE + (1 << 30), S0), "scale"),
    (lambda: fc.flse_mish_rows(FAKE, 4, 4, 4.0, 2.0, 1.0, FAKE + (1 << 30), S0), "cmin"),
    (lambda: fc.flse_mish_rows(FAKE, 4, 4, 4.0, -1.0, 1.0, FAKE + 8, S0), "overlaps"),
])
def test_epilogue_validation(call, frag):
    with pytest.raises(fc.FconvError) as e:
        call()
    assert e.value.code == fc.FCONV_EINVAL
    assert frag in e.value.message


def test_tensor_helpers_check_a_caller_supplied_out():
    """The tensor helpers pass `out` to kernels that write a fixed number of elements: a
    caller's buffer of another size, dtype or layout is rejected before any launch."""
    import torch
    cpu = torch.device("cpu")
    assert fc._prepare_out(None, (2, 3), cpu).shape == (2, 3)
    ok = torch.empty(6)
    assert fc._prepare_out(ok, (2, 3), cpu) is ok           # any shape with the right element count
    assert fc._prepare_out(torch.empty(4, 1), (4,), cpu) is not None
    for bad in (torch.empty(5), torch.empty(7), torch.empty(6, dtype=torch.float64),
                torch.empty(3, 4)[:, :2], torch.empty(6, device="meta")):
        with pytest.raises(ValueError, match="out must be"):
            fc._prepare_out(bad, (2, 3), cpu)


def test_tensor_helpers_need_one_device():
    import torch
    a, m = torch.empty(1), torch.empty(1, device="meta")
    assert fc._device_of(a, a, a) == a.device
    with pytest.raises(ValueError, match="one device"):
        fc._device_of(a, m)


@pytest.mark.gpu
def test_conv_helper_rejects_a_short_out_before_launch():
    import torch
    x = torch.zeros((1, 4, 8, 8), device="cuda")
    w = torch.zeros((8, 4, 3, 3), device="cuda")
    b = torch.zeros(8, device="cuda")
    short = torch.empty((1, 8, 6, 5), device="cuda")        # one column short of (1, 8, 6, 6)
    with pytest.raises(ValueError, match="out must be"):
        fc.conv_act_pool(x, w, b, act="gelu", pool=False, out=short)
    with pytest.raises(ValueError, match="out must be"):
        fc.gemm_lse_mish(torch.zeros((4, 8), device="cuda"), torch.zeros((3, 8), device="cuda"),
                         torch.zeros(3, device="cuda"), out=torch.empty(3, device="cuda"))


@pytest.mark.parametrize("dtype,iters,sink,frag", [
    (fc.DT_F32, 16, 0, "null"), (0x200, 16, FAKE, "dtype"), (fc.DT_BF16, 0, FAKE, "iters"),
    (fc.DT_F32, (1 << 20) + 1, FAKE, "iters"),
])
def test_mfma_rate_probe_validation(dtype, iters, sink, frag):
    with pytest.raises(fc.FconvError) as e:
        fc.fconv_mfma_rate_probe(dtype, iters, sink, S0)
    assert e.value.code == fc.FCONV_EINVAL and frag in e.value.message


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # pool partials of 512 x 64 x (28 x 7 tiles) x 4 B = 25.7 MB > the 16 MiB static scratch:
    # EINVAL before any HIP call
    with pytest.raises(fc.FconvError) as e:
        fc.fconv_act_pool_noalloc(FAKE, FAKE + (1 << 32), FAKE + (2 << 32), 512, 16, 224, 224, 64,
                                  fc.ACT_GELU, 1, FAKE + (3 << 32), S0)
    assert e.value.code == fc.FCONV_EINVAL and "scratch" in e.value.message


def test_noalloc_validates_like_the_allocating_entry_point():
    with pytest.raises(fc.FconvError) as e:
        fc.fconv_act_pool_noalloc(0, FAKE, FAKE, 2, 3, 16, 16, 8, fc.ACT_GELU, 1, FAKE, S0)
    assert e.value.code == fc.FCONV_EINVAL and "null" in e.value.message
