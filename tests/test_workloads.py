"""The seeded input generators: determinism, ranges and the recipe's structure."""
import numpy as np

import workloads as W


def test_layer_determinism_and_subset():
    a = W.draw_layer(5, E=8, H=64, I=32)
    b = W.draw_layer(5, E=8, H=64, I=32, experts=[6, 2])
    for p in ("gate", "up", "down"):
        pa, pb = getattr(a, p), getattr(b, p)
        assert np.array_equal(pa.codes[[2, 6]], pb.codes)
        assert np.array_equal(pa.scales[[2, 6]], pb.scales)
        assert np.array_equal(pa.gamma[[2, 6]], pb.gamma)
    assert b.slot(6) == 1 and a.slot(6) == 6
    assert a.gate.codes.shape == (8, 32, 32) and a.down.codes.shape == (8, 64, 16)
    assert a.gate.scales.shape == (8, 32, 4) and a.down.scales.shape == (8, 64, 2)


def test_scale_and_gamma_ranges():
    a = W.draw_layer(6, E=16, H=256, I=128)
    for p in (a.gate, a.up, a.down):
        assert p.scales.min() >= 0x18 and p.scales.max() <= 0x58
        assert len(np.unique(p.scales)) == 65
        g = p.gamma.astype(np.float64) * 2688.0
        assert np.all(g >= 0.5 - 1e-6) and np.all(g <= 2.0 + 1e-6)


def test_routing_and_weights():
    ids = W.draw_routing_uniform(1, 50)
    assert ids.shape == (50, 8) and all(len(set(r)) == 8 for r in ids)
    z = W.draw_routing_zipf(2, 4)
    assert all(len(set(r)) == 8 for r in z) and z.min() >= 0 and z.max() < 512
    u = len(np.unique(W.draw_workload(2).ids))
    assert 15 <= u <= 32
    w = W.draw_router_weights(3, 10)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6) and np.all(w > 0)
    big = W.draw_routing_zipf(4, 8192)
    cnt = np.bincount(big.reshape(-1), minlength=512)
    assert cnt.max() > 3000 and cnt.sum() == 8192 * 8


def test_activations_outliers():
    a = W.draw_activations(3, 64, 256)
    b = W.draw_activations(3, 64, 256, outlier_frac=0.01)
    fa = (a.astype(np.uint32) << 16).view(np.float32)
    fb = (b.astype(np.uint32) << 16).view(np.float32)
    diff = np.count_nonzero(fa != fb)
    assert diff <= round(0.01 * 64 * 256) and diff >= 0.9 * round(0.01 * 64 * 256)
    assert np.abs(fb).max() > 20


def test_linear_case():
    x, codes, scales, gamma = W.draw_linear_case(0)
    assert x.shape == (4, 128) and x.dtype == np.float32
    assert codes.shape == (64, 64) and scales.shape == (64, 8)
    assert gamma[0] == np.float32(1.0 / 2688.0)


def test_q8_0_down_layer():
    """Q8_0 down draws: shapes, all code bytes used, normal fp16 scales in [2^-14, 2^-12],
    unit gamma, the same bytes for a subset of experts, gate/up unchanged."""
    full = W.draw_layer(W.config_seed(2), E=6, H=64, I=96, down_fmt="q8_0")
    assert full.down.fmt == "q8_0" and full.gate.fmt == "nvfp4"
    assert full.down.codes.shape == (6, 64, 96) and full.down.codes.dtype == np.int8
    assert full.down.scales.shape == (6, 64, 3) and full.down.scales.dtype == np.uint16
    d = full.down.scales.view(np.float16).astype(np.float64)
    assert d.min() >= 2.0 ** -14 and d.max() <= 2.0 ** -12
    assert np.all(full.down.gamma == 1.0)
    sub = W.draw_layer(W.config_seed(2), E=6, H=64, I=96, experts=[4, 1], down_fmt="q8_0")
    assert np.array_equal(sub.down.codes[sub.slot(4)], full.down.codes[4])
    assert np.array_equal(sub.down.scales[sub.slot(1)], full.down.scales[1])
    nv = W.draw_layer(W.config_seed(2), E=6, H=64, I=96)
    assert np.array_equal(nv.gate.codes, full.gate.codes) and np.array_equal(nv.up.scales, full.up.scales)
    big = W.draw_layer(W.config_seed(2), E=1, H=256, I=256, down_fmt="q8_0")
    assert len(np.unique(big.down.codes)) == 256
