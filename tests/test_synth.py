"""Seeded input generator: determinism, published SplitMix64 outputs, moments, bf16 rounding."""
import json
import math
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64_seed0.json")))
    got = [format(int(v), "016x") for v in synth.splitmix64(g["seed"], 0, 3)]
    assert got == g["first_outputs_hex"]


def test_counter_based_offsets_agree():
    a = synth.splitmix64(1234, 0, 100)
    b = synth.splitmix64(1234, 37, 20)
    np.testing.assert_array_equal(a[37:57], b)


def test_deterministic_and_chunk_independent():
    a = synth.normal(99, (1 << 22) + 5)
    b = synth.normal(99, (1 << 22) + 5)
    np.testing.assert_array_equal(a, b)
    c = synth.normal(99, 1001)
    np.testing.assert_array_equal(a[:1001], c)
    u = synth.uniform(7, 3000, -0.5, 2.0)
    np.testing.assert_array_equal(u[:10], synth.uniform(7, 10, -0.5, 2.0))


def test_moments():
    n = 1 << 20
    x = synth.normal(5, n).astype(np.float64)
    assert abs(x.mean()) < 4 / math.sqrt(n)
    assert abs(x.var() - 1) < 4 * math.sqrt(2 / n)
    u = synth.uniform(6, n, -1.0, 1.0).astype(np.float64)
    assert u.min() >= -1 and u.max() < 1
    assert abs(u.mean()) < 4 * math.sqrt(1 / 3 / n)
    assert abs(u.var() - 1 / 3) < 0.01


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.0, 0.0], np.float32)
    bits = synth.to_bf16_bits(f)
    assert [hex(int(v)) for v in bits] == ["0x3f80", "0x3f80", "0x3f82", "0x3f81", "0xc000", "0x0"]
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(bits)[[0, 4, 5]], np.array([1.0, -2.0, 0.0], np.float32))


def test_workload_shapes_and_seeds_distinct():
    spec = synth.CONV_WORKLOADS["conv_tiny"]
    x, w, b = synth.conv_inputs(spec)
    assert x.shape == (2, 3, 16, 16) and w.shape == (8, 3, 3, 3) and b.shape == (8,)
    assert x.dtype == np.float32 and np.abs(x).max() <= 1
    assert np.abs(w).max() <= 1 / math.sqrt(27) and np.abs(b).max() <= 1 / math.sqrt(27)
    assert synth.seed_for(1, 0) != synth.seed_for(1, 1) != synth.seed_for(2, 0)
    small = dict(synth.CONV_WORKLOADS["conv_gelu_pool_bf16"], N=1, Cin=4, H=5, W=5, Cout=3)
    xb, wb, bb = synth.conv_inputs(small)
    assert xb.dtype == np.uint16 and wb.dtype == np.uint16 and bb.dtype == np.float32
