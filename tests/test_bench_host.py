"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic FLOP and byte
counts that the roofline fraction divides by, and the rule that an HBM traffic summary
counts only while the kernel sources it was measured on are unchanged."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    # the guard runs before torch is imported or any device is touched
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_conv_counts_fp32_pooled():
    # 64 x 16 x 224^2 -> 64, 3x3 valid: 222^2 outputs per (n, oc), 16 * 9 MACs each;
    # bytes: x and w once, the bias, the pooled (64, 64) result
    s = synth.CONV_WORKLOADS["conv_gelu_pool_f32"]
    assert bench.conv_flops(s) == 2 * 64 * 64 * 222 * 222 * 16 * 9
    assert bench.conv_bytes(s) == 4 * (64 * 16 * 224 * 224 + 64 * 16 * 9) + 4 * 64 + 4 * 64 * 64


def test_conv_counts_full_map():
    # 32 x 64 x 192^2 -> 128 with the whole (32, 128, 190, 190) fp32 map written
    s = synth.CONV_WORKLOADS["conv_mish2_full_f32"]
    assert bench.conv_flops(s) == 2 * 32 * 128 * 190 * 190 * 64 * 9
    assert bench.conv_bytes(s) == (4 * (32 * 64 * 192 * 192 + 128 * 64 * 9) + 4 * 128
                                   + 4 * 32 * 128 * 190 * 190)


def test_conv_counts_strided_padded_bf16():
    # 3x3, stride 2, padding 1 on 128^2: (128 + 2 - 3) // 2 + 1 = 64 outputs per side;
    # bf16 x and w (2 bytes), fp32 bias and pooled output
    s = synth.CONV_WORKLOADS["conv3x3_s2_gelu_pool_bf16"]
    assert bench.conv_flops(s) == 2 * 16 * 256 * 64 * 64 * 128 * 9
    assert bench.conv_bytes(s) == 2 * (16 * 128 * 128 * 128 + 256 * 128 * 9) + 4 * 256 + 4 * 16 * 256


def test_gemm_counts():
    s = synth.GEMM_WORKLOADS["gemm_lse_mish_f32"]
    assert bench.gemm_flops(s) == 2 * 2048 * 4096 * 6144
    assert bench.gemm_bytes(s) == 4 * (2048 * 4096 + 6144 * 4096) + 4 * (6144 + 2048)


def test_epilogue_bytes():
    s = synth.EPILOGUE_WORKLOADS["epi_mish2_f32"]
    n = 64 * 128 * 254 * 254
    assert s["shape"] == (64, 128, 254, 254)
    assert bench.epilogue_bytes(s) == 8 * n  # read once, written once


def test_traffic_summary_tied_to_kernel_sources(tmp_path, monkeypatch):
    kernel, wl = "gemm_lse_partials", "gemm_lse_mish_f32"
    for rel in bench.KERNEL_SOURCES[kernel]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic(wl, kernel) is None  # no summary
    prof = tmp_path / "profiles"
    prof.mkdir()
    summary = prof / f"{kernel}_{wl}.traffic.txt"
    summary.write_text(f"# header\nsource_hash: {bench.source_hash(kernel)}\nhbm_bytes_per_launch: 123456.0\n")
    assert bench.read_traffic(wl, kernel) == 123456.0
    # any change to a source the kernel is built from voids the summary
    src = tmp_path / bench.KERNEL_SOURCES[kernel][0]
    src.write_bytes(src.read_bytes() + b"\n")
    assert bench.read_traffic(wl, kernel) is None


def test_committed_traffic_summaries_are_well_formed():
    # every committed summary names a known kernel and workload and carries the fields
    # bench.py reads (whether its hash is current depends on the sources in the tree)
    names = sorted(f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith(".traffic.txt"))
    assert names
    workloads = set(synth.CONV_WORKLOADS) | set(synth.GEMM_WORKLOADS) | set(synth.EPILOGUE_WORKLOADS)
    for f in names:
        kernel = next(k for k in bench.KERNEL_SOURCES if f.startswith(k + "_"))
        wl = f[len(kernel) + 1:-len(".traffic.txt")]
        assert wl in workloads, f
        fields = dict(line.split(":", 1) for line in open(os.path.join(ROOT, "profiles", f))
                      if ":" in line and not line.startswith("#"))
        assert len(fields["source_hash"].strip()) == 16, f
        assert float(fields["hbm_bytes_per_launch"]) > 0, f


def test_default_run_covers_every_baseline_configuration():
    # the default line's headline plus its "configs" object are the five baseline
    # configurations: the tiny conv, the three full-size convs and the GEMM-LSE
    assert bench.DEFAULT_WORKLOAD == "baseline"
    names = [bench.HEADLINE] + bench.BASELINE_OTHERS
    cfgs = sorted(synth.CONV_WORKLOADS[n]["cfg"] if n in synth.CONV_WORKLOADS else synth.GEMM_WORKLOADS[n]["cfg"]
                  for n in names)
    assert cfgs == [1, 2, 3, 4, 5]
    assert len(set(names)) == 5
