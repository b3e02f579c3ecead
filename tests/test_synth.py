"""The synthetic-input generator: its mixer against SplitMix64's published vectors, slice
regeneration, thread-count independence and the recipes' value ranges (CPU only)."""
import json
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_vectors():
    ex = json.load(open(os.path.join(GOLD, "splitmix64_vectors.json")))
    s = ex["state"]
    out = []
    for _ in range(len(ex["outputs"])):
        s = (s + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
        out.append(str(synth.mix64(s)))
    assert out == ex["outputs"]


def test_slices_regenerate_and_threads_do_not_matter():
    full = synth.fill(synth.K_UNIT_ROWS, 5, 2, (100, 3, 16), "f32", row_len=16, threads=1)
    part = synth.fill(synth.K_UNIT_ROWS, 5, 2, (20, 3, 16), "f32", offset=40 * 3 * 16, row_len=16, threads=4)
    np.testing.assert_array_equal(full[40:60], part)
    a = synth.fill(synth.K_NORMAL, 9, 3, (50000,), "bf16", p0=1.0, threads=1)
    b = synth.fill(synth.K_NORMAL, 9, 3, (50000,), "bf16", p0=1.0, threads=7)
    np.testing.assert_array_equal(a, b)


def test_recipes_ranges():
    n = synth.fill(synth.K_NORMAL, 1, 1, (200000,), "f64", p0=1.0)
    assert abs(n.mean()) < 0.01 and abs(n.std() - 1) < 0.01
    u = synth.fill(synth.K_UNIT_ROWS, 1, 2, (1000, 128), "f64", row_len=128)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), 1, rtol=1e-14)
    s = synth.fill(synth.K_SIGMOID_NORMAL, 1, 4, (10000,), "f64")
    assert s.min() > 0 and s.max() < 1
    g = synth.fill(synth.K_LOGDECAY_SOFTPLUS, 1, 5, (10000,), "f64", p0=0.1)
    assert g.max() < 0 and g.min() > -1.0
    r = synth.fill(synth.K_LOGDECAY_RATE, 1, 5, (64, 4, 8), "f64", row_len=8, heads=4, p0=0.001, p1=0.1, tid2=7)
    assert r.max() < 0
    # per-(head, channel) rate: ratio to softplus draw is constant over tokens
    sp = -synth.fill(synth.K_LOGDECAY_SOFTPLUS, 1, 5, (64, 4, 8), "f64", p0=1.0)
    rate = -r / sp
    assert np.allclose(rate, rate[0:1], rtol=1e-12) and rate.min() > 0.001 - 1e-12 and rate.max() < 0.1
    L = synth.fill(synth.K_UNIFORM_INT, 1, 8, (5000,), "f64", p0=1024, p1=32768)
    assert L.min() >= 1024 and L.max() <= 32768 and np.all(L == np.floor(L))


def test_bf16_rounding_is_nearest_even():
    x = synth.fill(synth.K_NORMAL, 3, 3, (4096,), "f32", p0=1.0)
    b = synth.fill(synth.K_NORMAL, 3, 3, (4096,), "bf16", p0=1.0)
    wide = synth.bf16_bits_to_f32(b)
    # every bf16 value is the nearest representable to the fp32 value
    up = synth.bf16_bits_to_f32(b + 1)
    dn = synth.bf16_bits_to_f32(b - 1)
    err = np.abs(wide.astype(np.float64) - x)
    assert np.all(err <= np.abs(up.astype(np.float64) - x)) and np.all(err <= np.abs(dn.astype(np.float64) - x))


def test_workloads_shapes():
    w = synth.workload("varlen")
    assert len(w.lengths) == 8 and all(1024 <= L <= 32768 for L in w.lengths) and w.T == sum(w.lengths)
    w = synth.workload("tiny")
    q, k, v, g, b = synth.gen_tokens(w, w.T)
    assert q.shape == (64, 2, 16) and q.dtype == np.float32 and b.shape == (64, 2)
    assert synth.gen_state(w, 1) is None
