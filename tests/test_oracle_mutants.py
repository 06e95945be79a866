"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks that
the pins in test_oracle.py catch every one of them.

Each mutant is a one-token slip of the kind the pins are meant to catch: a
flipped or transposed kernel, a dropped bias, a wrong GELU constant or sign, a
single instead of double Mish, a wrong pool divisor, a missing max shift in
the logsumexp, the bias applied after the scale, a transposed GEMM operand, or
a missing factor in z * mish(z). The unmutated copy, built the same way, must
pass, so a failure really comes from the planted slip.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "kernel_flip": ("(ow + kw);", "(ow + 2 - kw);"),
    "kh_kw_swapped_in_w": ("* 3 + kh) * 3 + kw;", "* 3 + kw) * 3 + kh;"),
    "channels_reversed": ("((size_t)n * Cin + ic) * H", "((size_t)n * Cin + (Cin - 1 - ic)) * H"),
    "dropped_bias": ("return acc + (double)b[oc];", "return acc;"),
    "gelu_wrong_constant": ("erf(v / sqrt(2.0))", "erf(v / 2.0)"),
    "gelu_wrong_sign": ("(1.0 + erf(", "(1.0 - erf("),
    "gelu_tanh_no_cubic": ("(v + 0.044715 * v * v * v)", "(v)"),
    "gelu_tanh_wrong_constant": ("0.044715", "0.04715"),
    "gelu_tanh_half_dropped": ("return 0.5 * v * (1.0 + tanh(", "return v * (1.0 + tanh("),
    "conv2d_stride_ignored": ("int ih = oh * S + kh - P;", "int ih = oh + kh - P;"),
    "conv2d_padding_sign": ("int iw = ow * S + kw - P;", "int iw = ow * S + kw + P;"),
    "conv2d_padding_clamped": ("if (ih < 0 || ih >= H) continue; /* zero padding */",
                               "if (ih < 0) ih = 0; if (ih >= H) ih = H - 1;"),
    "conv2d_out_size": ("*OH = (H + 2 * P - K) / S + 1;", "*OH = (H + 2 * P - K) / S;"),
    "softplus_wrong_sign": ("log1p(exp(-fabs(v)))", "log1p(exp(fabs(v)))"),
    "single_mish": ("return oracle_mish(oracle_mish(v));", "return oracle_mish(v);"),
    "pool_divisor_full_map": ("((double)OH * (double)OW)", "((double)H * (double)W)"),
    "lse_missing_shift": ("double z = mx + log(s);", "double z = log(s);"),
    "bias_after_scale": ("scale * (dot + (double)b[j])", "scale * dot + (double)b[j]"),
    "gemm_w_transposed": ("load_elem(Wt, (size_t)j * K + k, dtype)", "load_elem(Wt, (size_t)k * N + j, dtype)"),
    "gemm_w_read_as_float32": ("load_elem(Wt, (size_t)j * K + k, dtype)", "load_elem(Wt, (size_t)j * K + k, 0)"),
    "out_missing_z_factor": ("out[i] = z * oracle_mish(z);", "out[i] = oracle_mish(z);"),
    "act_mean_wrong_divisor": ("return s / (double)count;", "return s / (double)(count + 1);"),
    "lse_rows_scale_dropped": ("c[j] = fmin(fmax(scale * (double)r[j], cmin), cmax);",
                               "c[j] = fmin(fmax((double)r[j], cmin), cmax);"),
    "lse_rows_missing_z_factor": ("out[m] = z * oracle_mish(z);", "out[m] = oracle_mish(z);"),
}


def _build(src_text, path):
    with open(path + ".c", "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-fno-fast-math",
                    "-ffp-contract=off", path + ".c", "-o", path, "-lm"], check=True)


def _run_pins(lib):
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], env=env, cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=300)
    return r.returncode, r.stdout.decode(errors="replace")[-2000:]


def test_every_planted_mistake_is_caught():
    src = open(SRC).read()
    with tempfile.TemporaryDirectory() as d:
        libs = {"control": os.path.join(d, "control.so")}
        _build(src, libs["control"])
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) >= 1, f"mutation site for {name} absent"
            libs[name] = os.path.join(d, name + ".so")
            _build(src.replace(old, new), libs[name])
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            results = dict(zip(libs, ex.map(_run_pins, libs.values())))
    rc, log = results.pop("control")
    assert rc == 0, "unmutated oracle copy failed its pins:\n" + log
    survivors = [name for name, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"
