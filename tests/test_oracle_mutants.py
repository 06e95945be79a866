"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks that
the pins in test_oracle.py catch every one of them.

Each mutant is a one-token slip of the kind the pins are meant to catch: a
flipped or transposed kernel, a dropped bias, a wrong GELU constant or sign, a
single instead of double Mish, a wrong pool divisor, a missing max shift or log
term in the logsumexp, the bias applied after the scale, a transposed GEMM
operand, or a missing factor in z * mish(z).

Every mutant edits exactly ONE site. A slip pattern that occurs in several
functions of the oracle (the logsumexp line appears in three of them) becomes
one mutant per occurrence, named after the function it lands in, so a slip that
one function's pins miss cannot hide behind the same slip caught in another.
The test also requires that every function doing arithmetic of the method has
at least one planted slip, and prints the kills per function. The unmutated
copy, built the same way, must pass, so a failure really comes from the slip.
"""
import concurrent.futures
import os
import re
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# slip name -> (text at the site, replacement); expanded to one mutant per occurrence
SLIPS = {
    "bf16_widen_shift": ("((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    "kernel_flip": ("(ow + kw);", "(ow + 2 - kw);"),
    "kh_kw_swapped_in_w": ("* 3 + kh) * 3 + kw;", "* 3 + kw) * 3 + kh;"),
    "channels_reversed": ("((size_t)n * Cin + ic) * H", "((size_t)n * Cin + (Cin - 1 - ic)) * H"),
    "dropped_bias": ("return acc + (double)b[oc];", "return acc;"),
    "gelu_wrong_constant": ("erf(v / sqrt(2.0))", "erf(v / 2.0)"),
    "gelu_wrong_sign": ("(1.0 + erf(", "(1.0 - erf("),
    "gelu_tanh_no_cubic": ("(v + 0.044715 * v * v * v)", "(v)"),
    "gelu_tanh_wrong_constant": ("0.044715", "0.04715"),
    "gelu_tanh_half_dropped": ("return 0.5 * v * (1.0 + tanh(", "return v * (1.0 + tanh("),
    "conv_full_map_nc_order": ("int n = (int)(nc / Cout), oc = (int)(nc % Cout);",
                               "int oc = (int)(nc / N), n = (int)(nc % N);"),
    "conv_pool_nc_order": ("int n = (int)(t / Cout), oc = (int)(t % Cout);",
                           "int oc = (int)(t / N), n = (int)(t % N);"),
    "conv2d_stride_ignored": ("int ih = oh * S + kh - P;", "int ih = oh + kh - P;"),
    "conv2d_padding_sign": ("int iw = ow * S + kw - P;", "int iw = ow * S + kw + P;"),
    "conv2d_padding_clamped": ("if (ih < 0 || ih >= H) continue; /* zero padding */",
                               "if (ih < 0) ih = 0; if (ih >= H) ih = H - 1;"),
    "conv2d_out_size": ("*OH = (H + 2 * P - K) / S + 1;", "*OH = (H + 2 * P - K) / S;"),
    "conv2d_kh_kw_swapped_in_w": ("* K + kh) * K + kw;", "* K + kw) * K + kh;"),
    "softplus_wrong_sign": ("log1p(exp(-fabs(v)))", "log1p(exp(fabs(v)))"),
    "mish_tanh_dropped": ("return v * tanh(oracle_softplus(v));", "return v * oracle_softplus(v);"),
    "single_mish": ("return oracle_mish(oracle_mish(v));", "return oracle_mish(v);"),
    "pool_divisor_full_map": ("((double)OH * (double)OW)", "((double)H * (double)W)"),
    "lse_missing_shift": ("double z = mx + log(s);", "double z = log(s);"),
    "lse_dropped_log_sum": ("double z = mx + log(s);", "double z = mx;"),
    "lse_gemm_sum_unshifted": ("s += exp(c[j] - mx);", "s += exp(c[j]);"),
    "lse_rows_sum_unshifted": ("s += exp(r[j] - mx);", "s += exp(r[j]);"),
    "lse_rows_max_not_taken": ("if (r[j] > mx) mx = r[j];", "if (r[j] < mx) mx = r[j];"),
    "bias_after_scale": ("scale * (dot + (double)b[j])", "scale * dot + (double)b[j]"),
    "gemm_clamp_bounds_swapped": ("c[j] = fmin(fmax(scale * (dot + (double)b[j]), cmin), cmax);",
                                  "c[j] = fmin(fmax(scale * (dot + (double)b[j]), cmax), cmin);"),
    "gemm_w_transposed": ("load_elem(Wt, (size_t)j * K + k, dtype)", "load_elem(Wt, (size_t)k * N + j, dtype)"),
    "gemm_w_read_as_float32": ("load_elem(Wt, (size_t)j * K + k, dtype)", "load_elem(Wt, (size_t)j * K + k, 0)"),
    "out_missing_z_factor": ("out[i] = z * oracle_mish(z);", "out[i] = oracle_mish(z);"),
    "rows_out_missing_z_factor": ("out[m] = z * oracle_mish(z);", "out[m] = oracle_mish(z);"),
    "act_mean_wrong_divisor": ("return s / (double)count;", "return s / (double)(count + 1);"),
    "act_pool_map_plane_offset": ("oracle_act_mean(x + p * hw, hw, act)", "oracle_act_mean(x + p, hw, act)"),
    "act_elementwise_act_dropped": ("out[i] = oracle_act((double)x[i], act);", "out[i] = (double)x[i];"),
    "lse_rows_scale_dropped": ("c[j] = fmin(fmax(scale * (double)r[j], cmin), cmax);",
                               "c[j] = fmin(fmax((double)r[j], cmin), cmax);"),
}

# Every function that does arithmetic of the method must carry at least one slip
# (argument-checking and thread-count helpers do none).
MUST_BE_MUTATED = {
    "widen_bf16", "oracle_softplus", "oracle_mish", "oracle_gelu", "oracle_gelu_tanh", "oracle_act",
    "conv_pre", "conv_pool_one", "oracle_conv_act_pool", "conv2d_pre", "conv2d_geometry", "conv2d_pool_one",
    "oracle_conv2d_act_pool", "oracle_gemm_lse_mish", "oracle_lse_mish_rows", "oracle_act_mean",
    "oracle_act_pool_map", "oracle_act_elementwise", "oracle_scale_clamp_lse_mish",
}

_FUNC_RE = re.compile(r"^(?:static\s+)?(?:double|int|void)\s+(\w+)\(", re.M)


def _function_at(src, offset):
    name = None
    for m in _FUNC_RE.finditer(src):
        if m.start() > offset:
            break
        name = m.group(1)
    return name


def _in_comment(src, offset):
    for m in re.finditer(r"/\*.*?\*/|//[^\n]*", src, re.S):
        if m.start() <= offset < m.end():
            return True
    return False


def expand_mutants(src):
    """{mutant id: (function, mutated source)}, one per occurrence of each slip's site in
    code (sites inside comments are skipped: editing them changes nothing)."""
    out = {}
    for slip, (old, new) in SLIPS.items():
        starts = [m.start() for m in re.finditer(re.escape(old), src) if not _in_comment(src, m.start())]
        assert starts, f"mutation site for {slip} absent"
        per_func = {}
        for at in starts:
            fn = _function_at(src, at)
            k = per_func.get(fn, 0)
            per_func[fn] = k + 1
            mid = f"{slip}@{fn}" + (f"#{k}" if k else "")
            out[mid] = (fn, src[:at] + new + src[at + len(old):])
    return out


def _build(src_text, path):
    with open(path + ".c", "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-fno-fast-math",
                    "-ffp-contract=off", path + ".c", "-o", path, "-lm"], check=True)


def _run_pins(lib):
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], env=env, cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=300)
    return r.returncode, r.stdout.decode(errors="replace")[-2000:]


def test_every_mutant_edits_one_site():
    src = open(SRC).read()
    for mid, (fn, text) in expand_mutants(src).items():
        assert fn is not None and text != src, mid
        # the original and the mutant differ in one stretch, which lies in code of the
        # function the mutant is named after
        i = len(os.path.commonprefix([src, text]))
        j = len(os.path.commonprefix([src[::-1], text[::-1]]))
        old, new = SLIPS[mid.split("@")[0]]
        assert len(src) - i - j <= len(old) and len(text) - i - j <= len(new), mid
        assert _function_at(src, i) == fn and not _in_comment(src, i), mid


def test_every_planted_mistake_is_caught():
    src = open(SRC).read()
    mutants = expand_mutants(src)
    funcs = {fn for fn, _ in mutants.values()}
    missing = MUST_BE_MUTATED - funcs
    assert not missing, f"functions with no planted slip: {sorted(missing)}"
    with tempfile.TemporaryDirectory() as d:
        libs = {"control": os.path.join(d, "control.so")}
        _build(src, libs["control"])
        for mid, (_, text) in mutants.items():
            libs[mid] = os.path.join(d, mid.replace("@", "_at_").replace("#", "_") + ".so")
            _build(text, libs[mid])
        workers = max(1, min(6, (os.cpu_count() or 2) - 1))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            results = dict(zip(libs, ex.map(_run_pins, libs.values())))
    rc, log = results.pop("control")
    assert rc == 0, "unmutated oracle copy failed its pins:\n" + log
    kills = {}
    for mid, (rc, _) in results.items():
        fn = mutants[mid][0]
        k, n = kills.get(fn, (0, 0))
        kills[fn] = (k + (rc != 0), n + 1)
    print("\nmutants caught per oracle function:")
    for fn in sorted(kills):
        print(f"  {fn:32s} {kills[fn][0]}/{kills[fn][1]}")
    survivors = [mid for mid, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"
