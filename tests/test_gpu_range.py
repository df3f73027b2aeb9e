"""Operand range and non-finite values, prefill and decode, against the float64 oracle.

The prefill GEMMs take fp16 operands. Each token row of x, and each routed pair's h per
block of intermediate indices, carries a power-of-two exponent that is undone exactly at
the FP32 accumulator, so activations far outside fp16's range give the oracle's result
("Strata NVFP4" README, "How it differs from upstream Strata": the scale fold that left
hidden activations in FP16 subnormals and cost 2-12% expert error). NaN and infinite
activations or scale bytes give NaN exactly where the float64 definition does (the
reading that non-finite values propagate)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, bf16_dev, layer_dev, max_row_rel_l2

pytestmark = pytest.mark.gpu
nv = pytest.importorskip("nvfp4_quantized_moe_02_amd")

E, H, I, T, K = 8, 512, 256, 200, 4


def _case(seed=61):
    lay = W.draw_layer(seed, E=E, H=H, I=I)
    ids = W.draw_routing_zipf(seed, T, E, K)
    w = W.draw_router_weights(seed, T, K)
    x = np.random.default_rng(seed).standard_normal((T, H)).astype(np.float32)
    return lay, ids, w, x


def _scaled(x):
    """Rows 0..49 times 1e5 (h near 1e7, past fp16's 65504), rows 50..99 times 1e-6 (h near
    1e-15, below fp16's smallest subnormal), rows 100..119 with one element times 1e12 and
    the rest normal (a row whose range exceeds fp16's), the rest unchanged."""
    x = x.copy()
    x[:50] *= 1e5
    x[50:100] *= 1e-6
    x[100:120, 7] *= 1e12
    return x


def _run(kind, lay, dl, xb, ids, w, act="bf16"):
    ti, tw = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    if kind == "prefill":
        y = nv.moe_prefill(bf16_dev(xb), dl, ti, tw, act=act, out_dtype=torch.float32)
    else:
        y = torch.cat([nv.moe_decode(bf16_dev(xb[t:t + 8]), dl, ti[t:t + 8], tw[t:t + 8])
                       for t in range(0, xb.shape[0], 8)])
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_activations_far_outside_fp16_range(kind):
    lay, ids, w, x = _case()
    dl = layer_dev(lay)
    xb = W.f32_to_bf16_bits(_scaled(x))
    got = _run(kind, lay, dl, xb, ids, w)
    ref = O.moe_grouped(O.bf16_to_f64(xb), lay, ids, w)
    assert np.isfinite(ref).all() and np.isfinite(got).all()
    err = O.rel_l2_rows(got, ref)
    print(f"{kind}: max row rel L2, rows x1e5 {err[:50].max():.2e}, x1e-6 {err[50:100].max():.2e}, "
          f"one element x1e12 {err[100:120].max():.2e}, others {err[120:].max():.2e}")
    bar = 5e-4 if kind == "prefill" else 1e-5  # fp16 h rounding (prefill); FP32 only (decode)
    assert err.max() < bar


def test_prefill_range_beats_plain_fp16():
    """On those rows h itself leaves fp16's range: past 65504 on a x1e5 row, below the
    smallest fp16 subnormal (2^-24) on a x1e-6 row, so plain fp16 operands would overflow
    or vanish and the check above is not vacuous."""
    lay, ids, w, x = _case()
    xs = O.bf16_to_f64(W.f32_to_bf16_bits(_scaled(x)))
    hmax = []
    for t in (0, 60):
        e = int(ids[t, 0])
        g = O.linear(xs[t:t + 1], lay.gate.codes[e], lay.gate.scales[e], lay.gate.gamma[e])
        u = O.linear(xs[t:t + 1], lay.up.codes[e], lay.up.scales[e], lay.up.gamma[e])
        hmax.append(float(np.abs(O.silu(g) * u).max()))
    assert hmax[0] > 65504 and hmax[1] < 2.0 ** -24, hmax


def test_prefill_w4a8_extreme_rows():
    """W4A8 on the same rows: int8 codes with fp32 row scales carry any range."""
    lay, ids, w, x = _case()
    dl = layer_dev(lay)
    xb = W.f32_to_bf16_bits(_scaled(x))
    got = _run("prefill", lay, dl, xb, ids, w, act="w4a8_f16")
    ref = O.moe_w4a8(xb, lay, ids, w)
    err = O.rel_l2_rows(got, ref)
    print(f"w4a8 extreme rows: max row rel L2 {err.max():.2e}")
    assert np.isfinite(got).all() and err.max() < 2e-2  # int8 rounding of h near ties included


@pytest.mark.parametrize("kind", ["prefill", "decode"])
@pytest.mark.parametrize("where", ["gate", "down", "x_inf", "x_nan"])
def test_nonfinite_propagates_where_the_oracle_has_nan(kind, where):
    lay, ids, w, x = _case(67)
    e = int(ids[3, 0])
    if where == "gate":
        lay.gate.scales[e, 5, 3] = 0x7F   # NaN scale byte: g[5] is NaN for every pair of e
    elif where == "down":
        lay.down.scales[e, 9, 1] = 0xFF   # NaN (negative-sign pattern): output 9 of e's tokens
    elif where == "x_inf":
        x[11, 100] = np.inf
    else:
        x[12, 3] = np.nan
    dl = layer_dev(lay)
    xb = W.f32_to_bf16_bits(x)
    got = _run(kind, lay, dl, xb, ids, w)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = O.moe_grouped(O.bf16_to_f64(xb), lay, ids, w)
    nan_r = np.isnan(ref)
    assert nan_r.any()
    assert np.array_equal(np.isnan(got), nan_r), (np.argwhere(np.isnan(got) != nan_r)[:5])
    fin = ~nan_r.any(axis=1)
    bar = 5e-4 if kind == "prefill" else 1e-5
    assert max_row_rel_l2(got[fin], ref[fin]) < bar
