"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something it does not itself compute: value
tables of the element formats, a library decoder (torch.float8_e4m3fn), exact
rational brute force, closed forms, hand-derived fixtures under tests/golden/
and invariants of the method. A negative-control section plants plausible
mistakes in copies of oracle functions and checks that a pin catches each.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from conftest import read_golden


# ------------------------------------------------------------------ element formats
def _e2m1_golden():
    tab = {}
    for ln in read_golden("e2m1_values.txt"):
        c, v = ln.split()
        tab[int(c)] = float(v)
    return tab


def test_e2m1_table_matches_golden():
    tab = _e2m1_golden()
    assert sorted(tab) == list(range(16))
    got = O.e2m1_value(np.arange(16))
    for c in range(16):
        assert got[c] == tab[c]
        assert math.copysign(1.0, got[c]) == math.copysign(1.0, tab[c])  # -0 for code 8


def test_e4m3_all_bytes_match_torch_fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3fn_value(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3_spot_values_and_not_fnuz():
    for ln in read_golden("e4m3_spot_values.txt"):
        b, v = ln.split()
        got = float(O.e4m3fn_value(int(b, 16)))
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v), (b, got, v)
    fnuz = torch.tensor([0x38], dtype=torch.uint8).view(torch.float8_e4m3fnuz).to(torch.float64).item()
    assert fnuz == 0.5 and float(O.e4m3fn_value(0x38)) == 1.0


def test_pack_unpack_roundtrip_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    n = O.unpack_codes(b[None, :])[0]
    assert np.array_equal(n[0::2], b & 0xF) and np.array_equal(n[1::2], b >> 4)
    assert np.array_equal(O.pack_codes(n[None, :])[0], b)
    rng = np.random.default_rng(1)
    nib = rng.integers(0, 16, size=(7, 96), dtype=np.uint8)
    assert np.array_equal(O.unpack_codes(O.pack_codes(nib)), nib)


# ------------------------------------------------------------------ hand products
def _hand_cases():
    for ln in read_golden("hand_products.txt"):
        name, codes, scale, gamma, x, y = [f.strip() for f in ln.split("|")]
        cb = np.frombuffer(bytes.fromhex(codes), dtype=np.uint8)[None, :]
        sb = np.array([[int(scale, 16)]], dtype=np.uint8)
        xs = np.array([float(v) for v in x.split(",")])[None, :]
        yield name, cb, sb, float(gamma), xs, float(y)


@pytest.mark.parametrize("case", list(_hand_cases()), ids=lambda c: c[0])
def test_hand_products(case):
    name, cb, sb, gamma, xs, y = case
    assert O.linear(xs, cb, sb, gamma)[0, 0] == y


def test_global_scale_rounding_example():
    # code 7 (6.0) x scale 0x7E (448) x fp32(1/2688): exact product 1.0000000186264515,
    # which rounds to 1.0f in fp32 (one rounding).
    cb = np.array([[0x07] + [0] * 7], dtype=np.uint8)
    sb = np.array([[0x7E]], dtype=np.uint8)
    g = np.float32(1.0 / 2688.0)
    w64 = O.dequant(cb, sb, g)[0, 0]
    assert w64 == 6.0 * 448.0 * float(g)
    assert w64 == 1.0000000186264515
    assert O.dequant_f32(cb, sb, g)[0, 0] == np.float32(1.0)


def test_products_exact_in_bf16_and_f16():
    codes = np.arange(16)
    finite = [b for b in range(256) if (b & 0x7F) != 0x7F]
    v = O.e2m1_value(codes)[:, None] * O.e4m3fn_value(np.array(finite))[None, :]
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v)
    bf = O.bf16_to_f64(O.bf16_bits(v32))
    assert np.array_equal(bf, v)
    assert np.array_equal(v32.astype(np.float16).astype(np.float64), v)


# ------------------------------------------------------------------ brute force linear
def _frac_tables():
    e2 = {c: Fraction(v) for c, v in _e2m1_golden().items()}
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    e4 = {b: Fraction(float(t[b])) for b in range(256) if not math.isnan(t[b])}
    return e2, e4


def _bruteforce_linear(x, codes, scales, gamma):
    """Exact rational y[t][n] = gamma * sum_k x[t][k] * e2m1(code) * e4m3(scale),
    reading nibbles and groups straight from the bytes."""
    e2, e4 = _frac_tables()
    T, K = x.shape
    N = codes.shape[0]
    y = np.zeros((T, N))
    g = Fraction(float(np.float32(gamma)))
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                byte = int(codes[n, k // 2])
                c = (byte >> 4) if (k % 2) else (byte & 0xF)
                acc += Fraction(float(x[t, k])) * e2[c] * e4[int(scales[n, k // 16])]
            y[t, n] = float(acc * g)
    return y


def test_linear_bruteforce_exact():
    rng = np.random.default_rng(7)
    T, N, K = 3, 5, 48  # N != K and three groups: a transposed operand or a wrong group index fails
    x = rng.standard_normal((T, K)).astype(np.float32).astype(np.float64)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0x18, 0x59, size=(N, K // 16), dtype=np.uint8)
    gamma = np.float32(0.37)
    ref = _bruteforce_linear(x, codes, scales, gamma)
    got = O.linear(x, codes, scales, gamma)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-14 * np.abs(ref).max())


def test_linear_small_config_against_bruteforce():
    x, codes, scales, gamma = W.draw_linear_case(0)
    x = x.astype(np.float64)
    ref = _bruteforce_linear(x[:2], codes[:6], scales[:6], gamma[0])
    got = O.linear(x[:2], codes[:6], scales[:6], gamma[0])
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-13)


# ------------------------------------------------------------------ SiLU closed forms
def test_silu_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-16
    assert abs(O.silu(np.array([-1.0]))[0] + 0.2689414213699951) < 1e-16
    z = np.linspace(-30, 30, 121)
    # z*sigma(z) - (-z)*sigma(-z) = z for every z: a sign error in the exponent breaks it
    assert np.allclose(O.silu(z) - O.silu(-z), z, rtol=0, atol=1e-12)
    assert O.silu(np.array([800.0]))[0] == 800.0
    assert O.silu(np.array([-800.0]))[0] == 0.0


# ------------------------------------------------------------------ MoE
def _const_proj(E, N, K, code_byte, scale_byte, gammas):
    return W.Proj(np.full((E, N, K // 2), code_byte, np.uint8),
                  np.full((E, N, K // 16), scale_byte, np.uint8),
                  np.asarray(gammas, np.float32))


def test_moe_hand_closed_form():
    """E=2, H=I=16. Expert 0: gate codes 1.0, gamma 1/16 -> g = 1 for x = ones;
    up codes 2.0, gamma 1/4 -> u = 8; h = SiLU(1) * 8; down codes 1.0, gamma 1/32 ->
    y_n = 16 * h / 32. Expert 1: gate codes -1.0 (byte 0xAA), gamma 1/16 -> g = -1;
    up codes 0.5 (0x11), gamma 1 -> u = 8; down codes -2.0 (0xCC), gamma 1/64 ->
    y_n = -2 * 16 * SiLU(-1) * 8 / 64. Slot weights 0.75 and 0.25."""
    H = I = 16
    gate = W.Proj(np.stack([np.full((I, H // 2), 0x22, np.uint8), np.full((I, H // 2), 0xAA, np.uint8)]),
                  np.full((2, I, 1), 0x38, np.uint8), np.array([1 / 16, 1 / 16], np.float32))
    up = W.Proj(np.stack([np.full((I, H // 2), 0x44, np.uint8), np.full((I, H // 2), 0x11, np.uint8)]),
                np.full((2, I, 1), 0x38, np.uint8), np.array([1 / 4, 1.0], np.float32))
    down = W.Proj(np.stack([np.full((H, I // 2), 0x22, np.uint8), np.full((H, I // 2), 0xCC, np.uint8)]),
                  np.full((2, H, 1), 0x38, np.uint8), np.array([1 / 32, 1 / 64], np.float32))
    lay = W.Layer(gate, up, down, E=2, H=H, I=I)
    x = np.ones((1, H))
    ids = np.array([[0, 1]], np.int32)
    w = np.array([[0.75, 0.25]], np.float32)
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    sm1 = -1.0 / (1.0 + math.exp(1.0))
    y0 = 16 * (s1 * 8) / 32
    y1 = -2 * 16 * (sm1 * 8) / 64
    expect = 0.75 * y0 + 0.25 * y1
    for fn in (O.moe_pairwise, O.moe_grouped):
        out = fn(x, lay, ids, w)
        assert out.shape == (1, H)
        assert np.allclose(out, expect, rtol=1e-15, atol=0)


def _small_layer(seed=3, E=6, H=32, I=48):
    return W.draw_layer(seed, E=E, H=H, I=I)


def _compose_ffn(x, lay, e):
    """FFN built from the separately pinned pieces (linear, silu)."""
    g = O.linear(x, lay.gate.codes[e], lay.gate.scales[e], lay.gate.gamma[e])
    u = O.linear(x, lay.up.codes[e], lay.up.scales[e], lay.up.gamma[e])
    h = O.silu(g) * u
    return O.linear(h, lay.down.codes[e], lay.down.scales[e], lay.down.gamma[e])


def test_moe_single_expert_reduces_to_ffn():
    lay = _small_layer()
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, lay.H))
    for e in range(lay.E):
        ids = np.full((5, 1), e, np.int32)
        w = np.ones((5, 1), np.float32)
        ref = _compose_ffn(x, lay, e)
        assert np.allclose(O.moe_pairwise(x, lay, ids, w), ref, rtol=1e-13, atol=1e-13)


def test_pairwise_matches_grouped_and_invariants():
    lay = _small_layer()
    rng = np.random.default_rng(5)
    T, k = 9, 4
    x = rng.standard_normal((T, lay.H))
    ids = rng.integers(0, lay.E, size=(T, k)).astype(np.int32)
    ids[2, 1] = ids[2, 0]          # duplicate expert within a token
    ids[4, 3] = -1                 # dropped
    ids[6, 0] = lay.E + 3          # dropped
    w = rng.random((T, k)).astype(np.float32)
    a = O.moe_pairwise(x, lay, ids, w)
    b = O.moe_grouped(x, lay, ids, w)
    scale = np.abs(a).max()
    assert np.abs(a - b).max() <= 1e-12 * scale
    # slot permutation invariance
    perm = rng.permutation(k)
    c = O.moe_grouped(x, lay, ids[:, perm], w[:, perm])
    assert np.abs(a - c).max() <= 1e-12 * scale
    # linear in the router weights
    d = O.moe_grouped(x, lay, ids, (2 * w).astype(np.float32))
    assert np.abs(d - 2 * a).max() <= 1e-12 * scale
    # zero weights give zero
    assert not np.any(O.moe_grouped(x, lay, ids, np.zeros_like(w)))
    # dropped ids equal a zero weight on a valid id
    ids2, w2 = ids.copy(), w.copy()
    ids2[4, 3], w2[4, 3] = 0, 0.0
    ids2[6, 0], w2[6, 0] = 0, 0.0
    assert np.abs(O.moe_grouped(x, lay, ids2, w2) - a).max() <= 1e-12 * scale
    # duplicate ids sum: merging the two slots' weights into one gives the same
    ids3, w3 = ids.copy(), w.copy()
    w3[2, 0] = np.float32(w[2, 0] + w[2, 1])
    ids3[2, 1], w3[2, 1] = 0, 0.0
    row = O.moe_pairwise(x, lay, ids3, w3)[2]
    assert np.allclose(row, a[2], rtol=1e-6, atol=1e-9 * scale)


def test_moe_rows_subset():
    lay = _small_layer()
    rng = np.random.default_rng(9)
    x = rng.standard_normal((7, lay.H))
    ids = rng.integers(0, lay.E, size=(7, 3)).astype(np.int32)
    w = rng.random((7, 3)).astype(np.float32)
    full = O.moe_grouped(x, lay, ids, w)
    rows = [5, 1, 6]
    assert np.array_equal(O.moe_grouped(x, lay, ids, w, rows=rows), full[rows]) or \
        np.allclose(O.moe_grouped(x, lay, ids, w, rows=rows), full[rows], rtol=1e-14, atol=0)
    assert np.allclose(O.moe_pairwise(x, lay, ids, w, rows=rows), full[rows], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ routing
def test_route_matches_stable_sort():
    rng = np.random.default_rng(11)
    for T, k, E in [(1, 8, 512), (5, 3, 4), (37, 8, 16), (200, 2, 7)]:
        ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)
        off, sp = O.route(ids, E)
        flat = ids.reshape(-1)
        valid = [p for p in range(T * k) if 0 <= flat[p] < E]
        expect = sorted(valid, key=lambda p: flat[p])  # Python's sort is stable
        n = len(expect)
        assert off[0] == 0 and off[E] == n and np.all(np.diff(off) >= 0)
        assert list(sp[:n]) == expect and np.all(sp[n:] == -1)
        for e in range(E):
            assert np.all(flat[sp[off[e]:off[e + 1]]] == e)


# ------------------------------------------------------------------ W4A8 quantizer
def test_quant_i8_fixture():
    for ln in read_golden("quant_i8_cases.txt"):
        xs, s, q = [f.strip() for f in ln.split("|")]
        x = np.array([[float(v) for v in xs.split(",")]], dtype=np.float32)
        qq, ss = O.quant_rows_i8(x)
        want = np.float32(float(s))
        assert ss[0] == want or (np.isnan(want) and np.isnan(ss[0])), (xs, ss[0])
        assert list(qq[0]) == [int(v) for v in q.split(",")], (xs, qq[0])


def test_quant_i8_properties():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((64, 768)) * rng.uniform(1e-3, 1e3, size=(64, 1))).astype(np.float32)
    q, s = O.quant_rows_i8(x)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(64), am].astype(int)) == 127)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= 0.5 * s[:, None].astype(np.float64) * (1 + 1e-6))


def test_w4a8_ffn_composition():
    """W4A8 FFN = pinned pieces: quantize x, linear, silu, fp32 h, quantize h, linear."""
    lay = _small_layer(E=2)
    rng = np.random.default_rng(17)
    xb = W.f32_to_bf16_bits(rng.standard_normal((4, lay.H)).astype(np.float32))
    ids = np.array([[0], [1], [1], [0]], np.int32)
    w = np.ones((4, 1), np.float32)
    got = O.moe_w4a8(xb, lay, ids, w)
    x32 = O.bf16_to_f64(xb).astype(np.float32)
    qx, sx = O.quant_rows_i8(x32)
    xh = qx.astype(np.float64) * sx.astype(np.float64)[:, None]
    for t in range(4):
        e = ids[t, 0]
        g = O.linear(xh[t:t + 1], lay.gate.codes[e], lay.gate.scales[e], lay.gate.gamma[e])
        u = O.linear(xh[t:t + 1], lay.up.codes[e], lay.up.scales[e], lay.up.gamma[e])
        h = (O.silu(g) * u).astype(np.float32)
        qh, sh = O.quant_rows_i8(h)
        hh = qh.astype(np.float64) * float(sh[0])
        y = O.linear(hh, lay.down.codes[e], lay.down.scales[e], lay.down.gamma[e])
        assert np.allclose(got[t], y[0], rtol=1e-13, atol=1e-13 * np.abs(y).max())


def test_w4a8_exact_int8_inputs():
    """Activations that are exactly q * 2^-4 with |q| <= 127 and a 127 present
    quantize losslessly: the first GEMM equals the unquantized one."""
    rng = np.random.default_rng(19)
    q = rng.integers(-127, 128, size=(3, 32))
    q[:, 0] = 127
    x32 = (q * 0.0625).astype(np.float32)
    qq, s = O.quant_rows_i8(x32)
    assert np.all(s == np.float32(0.0625)) and np.array_equal(qq.astype(int), q)


def test_w4a8_nonfinite_rows_propagate():
    """A NaN or infinite activation makes its whole token row of the W4A8 output NaN
    (the quantizer's reading for non-finite rows); every other row stays finite."""
    lay = _small_layer(E=2)
    rng = np.random.default_rng(23)
    x = rng.standard_normal((4, lay.H)).astype(np.float32)
    x[1, 5] = np.nan
    x[2, 0] = np.inf
    xb = W.f32_to_bf16_bits(x)
    ids = np.array([[0, 1], [1, 0], [0, 1], [1, 0]], np.int32)
    w = np.full((4, 2), 0.5, np.float32)
    with np.errstate(invalid="ignore"):
        y = O.moe_w4a8(xb, lay, ids, w)
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all()
    assert np.isfinite(y[0]).all() and np.isfinite(y[3]).all()


def test_w4a8_down_from_codes_reproduces_moe_w4a8():
    """The down step on supplied int8 hidden codes, fed the oracle's own codes (from
    w4a8_pair_hidden, quantized), reproduces the pinned W4A8 composition; pinned the
    other way too: one flipped code moves exactly one output row, by w * s * gamma_d
    times one down column."""
    lay = _small_layer(seed=5, E=4)
    rng = np.random.default_rng(29)
    T, k = 6, 2
    xb = W.f32_to_bf16_bits(rng.standard_normal((T, lay.H)).astype(np.float32))
    ids = np.array([[0, 3], [3, 1], [2, 0], [1, 1], [0, -1], [3, 2]], np.int32)
    w = rng.random((T, k)).astype(np.float32)
    ref = O.moe_w4a8(xb, lay, ids, w)
    pairs, qs, ss = [], [], []
    for e, pe, h, s in O.w4a8_pair_hidden(xb, lay, ids):
        q, s2 = O.quant_rows_i8(h)
        assert np.array_equal(s2.view(np.uint32), s.view(np.uint32))
        pairs.append(pe)
        qs.append(q)
        ss.append(s2)
    pairs, qs, ss = np.concatenate(pairs), np.concatenate(qs), np.concatenate(ss)
    assert sorted(pairs.tolist()) == [p for p in range(T * k) if 0 <= ids.reshape(-1)[p] < lay.E]
    got = O.w4a8_down_from_codes(qs, ss, pairs, lay, ids, w)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    i, j = 3, 7
    qs2 = qs.copy()
    qs2[i, j] = qs2[i, j] + (1 if qs2[i, j] < 127 else -1)
    moved = O.w4a8_down_from_codes(qs2, ss, pairs, lay, ids, w) - got
    p = int(pairs[i])
    e = int(ids.reshape(-1)[p])
    Wd = O.dequant(lay.down.codes[e], lay.down.scales[e])
    expect = float(w.reshape(-1)[p]) * float(ss[i]) * float(lay.down.gamma[e]) * (qs2[i, j] - qs[i, j]) * Wd[:, j]
    assert np.allclose(moved[p // k], expect, rtol=1e-12, atol=1e-15)
    assert np.count_nonzero(np.delete(moved, p // k, axis=0)) == 0


# ------------------------------------------------------------------ comparison measure
def _rows(field):
    return np.array([[float(v) for v in r.split(",")] for r in field.split(";")])


def test_rel_l2_rows_fixture():
    for ln in read_golden("rel_l2_cases.txt"):
        y, ref, want = [f.strip() for f in ln.split("|")]
        got = O.rel_l2_rows(_rows(y), _rows(ref))
        assert np.allclose(got, [float(v) for v in want.split(",")], rtol=1e-15, atol=0), (ln, got)


# ------------------------------------------------------------------ dequant roundings
def test_dequant_double_rounding_fixture():
    """bf16 / fp16 dequantization with a global scale rounds twice (exact -> fp32 ->
    narrow); the hand-derived ties make a single rounding give other bits."""
    for ln in read_golden("dequant_double_rounding.txt"):
        dt, code, sb, gbits, want, single = [f.strip() for f in ln.split("|")]
        codes = np.full((1, 16), int(code) * 0x11, np.uint8)  # every nibble = code
        scales = np.full((1, 2), int(sb, 16), np.uint8)
        gamma = np.array([int(gbits, 16)], np.uint32).view(np.float32)[0]
        got = (O.dequant_bf16(codes, scales, gamma) if dt == "bf16"
               else O.dequant_f16(codes, scales, gamma).view(np.uint16))
        assert np.all(got == int(want, 16)), (ln, hex(int(got[0, 0])))
        assert int(want, 16) != int(single, 16)
        # the single rounding of the exact float64 product, done by hand (ties are
        # impossible here): it lands on the other neighbour
        exact = float(O.dequant(codes, scales, gamma)[0, 0])
        lo = float(np.array([int(want, 16) << (16 if dt == "bf16" else 0)], np.uint32).view(np.float32)[0]) \
            if dt == "bf16" else float(np.array([int(want, 16)], np.uint16).view(np.float16)[0])
        hi = float(np.array([int(single, 16) << 16], np.uint32).view(np.float32)[0]) if dt == "bf16" \
            else float(np.array([int(single, 16)], np.uint16).view(np.float16)[0])
        assert lo < exact < hi and exact - lo > hi - exact


# ------------------------------------------------------------------ slicing (TF-906)
def test_row_and_input_partitions_reassemble():
    """TensorFold pull 906: row cuts and input cuts at multiples of 16 keep codes,
    scale bytes and the global scale; reassembly recovers the original bytes, and
    the partial products over input cuts sum to the full product."""
    lay = _small_layer(E=1, H=64, I=48)
    codes, scales, g = lay.gate.codes[0], lay.gate.scales[0], lay.gate.gamma[0]
    N, K = 48, 64
    rows = [(0, 16), (16, 40), (40, 48)]
    cols = [(0, 16), (16, 48), (48, 64)]
    full = O.dequant(codes, scales, g)
    assert np.array_equal(np.concatenate([O.dequant(codes[a:b], scales[a:b], g) for a, b in rows]), full)
    parts = [(codes[:, a // 2:b // 2], scales[:, a // 16:b // 16]) for a, b in cols]
    assert np.array_equal(np.concatenate([p[0] for p in parts], axis=1), codes)
    assert np.array_equal(np.concatenate([p[1] for p in parts], axis=1), scales)
    assert np.array_equal(np.concatenate([O.dequant(c, s, g) for c, s in parts], axis=1), full)
    x = np.random.default_rng(2).standard_normal((3, K))
    y = O.linear(x, codes, scales, g)
    ysum = sum(O.linear(x[:, a:b], c, s, g) for (a, b), (c, s) in zip(cols, parts))
    assert np.allclose(ysum, y, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ negative controls
def test_negative_controls_are_caught(monkeypatch):
    """Plant mistakes in the oracle (on the CPU) and check a pin fails for each."""
    cases = list(_hand_cases())
    nib = [c for c in cases if c[0] == "nibble_low"][0]

    # 1) swapped nibble order
    def unpack_swapped(codes):
        codes = np.asarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
        out[..., 0::2] = codes >> 4
        out[..., 1::2] = codes & 0x0F
        return out
    monkeypatch.setattr(O.nvfp4_oracle, "unpack_codes", unpack_swapped)
    assert O.nvfp4_oracle.linear(nib[4], nib[1], nib[2], nib[3])[0, 0] != nib[5]
    monkeypatch.undo()

    # 2) group size 32 instead of 16: the brute force over three groups disagrees
    def dequant_g32(codes, scales, gamma=None):
        vals = O.E2M1_TABLE[O.unpack_codes(codes)]
        sc = O.E4M3_TABLE[np.asarray(scales)]
        sc = np.repeat(sc, 32, axis=-1)[..., :vals.shape[-1]]
        return vals * sc
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 48))
    codes = rng.integers(0, 256, size=(3, 24), dtype=np.uint8)
    scales = rng.integers(0x18, 0x59, size=(3, 3), dtype=np.uint8)
    ref = _bruteforce_linear(x, codes, scales, 1.0)
    bad = x @ dequant_g32(codes, scales).T
    assert not np.allclose(bad, ref, rtol=1e-6)

    # 3) gate's global scale applied after SiLU: the hand closed form disagrees
    def ffn_gamma_after(x, Wg, gg, Wu, gu, Wd, gd):
        h = O.silu(x @ Wg.T) * gg * ((x @ Wu.T) * gu)
        return (h @ Wd.T) * gd
    monkeypatch.setattr(O.nvfp4_oracle, "expert_ffn", ffn_gamma_after)
    with pytest.raises(AssertionError):
        test_moe_hand_closed_form()
    monkeypatch.undo()

    # 4) gate and up swapped
    def ffn_swapped(x, Wg, gg, Wu, gu, Wd, gd):
        return expert_ref(x, Wu, gu, Wg, gg, Wd, gd)
    expert_ref = O.nvfp4_oracle.expert_ffn
    monkeypatch.setattr(O.nvfp4_oracle, "expert_ffn", ffn_swapped)
    with pytest.raises(AssertionError):
        test_moe_hand_closed_form()
    monkeypatch.undo()

    # 5) an unstable routing order fails the stable-sort pin
    ids = np.array([[3, 1], [3, 0], [1, 3]], np.int32)
    off, sp = O.route(ids, 4)
    unstable = list(sp[:6])
    i3 = [i for i in range(6) if ids.reshape(-1)[unstable[i]] == 3]
    unstable[i3[0]], unstable[i3[-1]] = unstable[i3[-1]], unstable[i3[0]]
    expect = sorted(range(6), key=lambda p: ids.reshape(-1)[p])
    assert list(sp[:6]) == expect and unstable != expect

    # 6) rounding the quantizer's quotient in float64 (not fp32) fails the fixture
    x = np.array([[12.7, -6.35, 0.05, 0, 0, 0, 0, 0]], np.float32)
    s = np.float32(12.7) / np.float32(127)
    q64 = np.rint(x.astype(np.float64) / float(s))
    assert q64[0, 1] == -63 and O.quant_rows_i8(x)[0][0, 1] == -64

    # 7) the comparison measure normalized by ||y||, or summed over the wrong axis,
    #    fails its hand fixture
    def rel_by_y(y, ref):
        y, ref = np.asarray(y, float), np.asarray(ref, float)
        return np.sqrt(((y - ref) ** 2).sum(-1)) / np.sqrt((y ** 2).sum(-1))

    def rel_cols(y, ref):
        y, ref = np.asarray(y, float), np.asarray(ref, float)
        return np.sqrt(((y - ref) ** 2).sum(0)) / np.sqrt((ref ** 2).sum(0))
    for bad in (rel_by_y, rel_cols):
        monkeypatch.setattr(O, "rel_l2_rows", bad)
        with pytest.raises(AssertionError):
            test_rel_l2_rows_fixture()
        monkeypatch.undo()

    # 8) a single rounding of the exact product to bf16 fails the double-rounding fixture
    def dequant_bf16_single(codes, scales, gamma=None):
        v = O.dequant(codes, scales, gamma)
        m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
        r = np.ldexp(np.rint(m * 256.0), e - 8)  # 8 significant bits, ties to even
        return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    monkeypatch.setattr(O, "dequant_bf16", dequant_bf16_single)
    with pytest.raises(AssertionError):
        test_dequant_double_rounding_fixture()
    monkeypatch.undo()


# ------------------------------------------------------------------ Q8_0 down projection
def _fp16_value(bits):
    """IEEE binary16 value of a bit pattern, as an exact Fraction (by the definition)."""
    s, e, m = (bits >> 15) & 1, (bits >> 10) & 0x1F, bits & 0x3FF
    assert e != 0x1F
    v = Fraction(m, 1024) * Fraction(2) ** -14 if e == 0 else (1 + Fraction(m, 1024)) * Fraction(2) ** (e - 15)
    return -v if s else v


def test_q8_0_dequant_bruteforce_all_codes():
    """Every int8 code with normal, subnormal, negative and zero fp16 scales, against the
    exact rational product; scale b covers inputs 32b .. 32b+31."""
    scale_bits = [0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x1C00, 0x3C00, 0x3555, 0x7BFF, 0xBC00, 0xC4D2, 0x2E66]
    K = 256 * len(scale_bits)
    codes = np.tile(np.arange(-128, 128, dtype=np.int16), len(scale_bits))
    # element k takes scale k // 32: repeat each scale over 8 blocks of 32 = 256 codes
    scales = np.repeat(np.array(scale_bits, np.uint16), 8)
    got = O.dequant_q8_0(codes.astype(np.int8)[None], scales[None])[0]
    assert got.shape == (K,)
    for k in range(K):
        want = _fp16_value(int(scales[k // 32])) * int(codes[k])
        assert Fraction(got[k]) == want, (k, got[k], want)


def test_q8_0_layout_hand():
    """Hand example, K = 64: row 1, input 40 is code -3 with scale 2^-3 (block 1)."""
    codes = np.zeros((2, 64), np.int8)
    scales = np.zeros((2, 2), np.uint16)
    codes[1, 40], codes[1, 31], codes[0, 32] = -3, 7, 5
    scales[1] = [0x3C00, 0x3000]   # 1.0, 0.125
    scales[0] = [0x4000, 0x4400]   # 2.0, 4.0
    W_ = O.dequant_q8_0(codes, scales)
    assert W_[1, 40] == -0.375 and W_[1, 31] == 7.0 and W_[0, 32] == 20.0
    assert np.count_nonzero(W_) == 3


def _paired_nvfp4_and_q8(seed, E, N, K):
    """An NVFP4 projection whose two 16-groups of every 32-block share one E4M3 scale s,
    and the Q8_0 projection of the same real matrix: q = 2 * e2m1 (an integer in
    [-12, 12]) and d = s / 2 (exact in fp16)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    sb = rng.integers(0x18, 0x59, size=(E, N, K // 32), dtype=np.uint8)
    scales = np.repeat(sb, 2, axis=-1)
    nib = np.empty((E, N, K), np.int64)
    nib[..., 0::2] = codes & 0x0F
    nib[..., 1::2] = codes >> 4
    mag = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64)           # 2 * |e2m1|
    q = np.where(nib & 8, -mag[nib & 7], mag[nib & 7]).astype(np.int8)
    half = np.array([float(_e4m3_frac(int(b)) / 2) for b in range(256)])
    d = half[sb].astype(np.float16)
    assert np.array_equal(d.astype(np.float64), half[sb])          # s / 2 is exact in fp16
    return codes, scales, q, d.view(np.uint16)


def _e4m3_frac(b):
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def test_q8_0_down_equals_nvfp4_down_on_the_same_matrix():
    """The MoE with a Q8_0 down projection equals the (separately pinned) NVFP4 MoE when
    both hold the same real matrix."""
    lay = W.draw_layer(4, E=5, H=64, I=96)
    codes, scales, q, d = _paired_nvfp4_and_q8(11, lay.E, lay.H, lay.I)
    lay.down = W.Proj(codes, scales, lay.down.gamma)
    lay8 = W.Layer(lay.gate, lay.up, W.Q8Proj(q, d, lay.down.gamma.copy()), lay.E, lay.H, lay.I)
    assert np.array_equal(O.dequant(codes, scales), O.dequant_q8_0(q, d))
    rng = np.random.default_rng(12)
    T, k = 7, 3
    x = rng.standard_normal((T, lay.H))
    ids = rng.integers(0, lay.E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    a = O.moe_pairwise(x, lay, ids, w)
    b = O.moe_pairwise(x, lay8, ids, w)
    c = O.moe_grouped(x, lay8, ids, w)
    assert np.array_equal(a, b)
    assert np.abs(c - a).max() <= 1e-12 * np.abs(a).max()


def test_q8_0_negative_controls(monkeypatch):
    """Plausible mistakes in the Q8_0 decoder fail the pins above."""
    def unsigned_codes(codes, scales):
        q = np.asarray(codes).view(np.uint8).astype(np.float64)
        dd = np.asarray(scales, np.uint16).view(np.float16).astype(np.float64)
        return q * np.repeat(dd, 32, axis=-1)
    def block16(codes, scales):
        q = np.asarray(codes, np.int8).astype(np.float64)
        dd = np.asarray(scales, np.uint16).view(np.float16).astype(np.float64)
        return q * np.repeat(dd, 16, axis=-1)[..., :q.shape[-1]]
    def bf16_scales(codes, scales):
        q = np.asarray(codes, np.int8).astype(np.float64)
        dd = (np.asarray(scales, np.uint32) << 16).view(np.float32).astype(np.float64)
        return q * np.repeat(dd, 32, axis=-1)
    for bad in (unsigned_codes, block16, bf16_scales):
        monkeypatch.setattr(O.nvfp4_oracle, "dequant_q8_0", bad)
        monkeypatch.setattr(O, "dequant_q8_0", bad)
        with pytest.raises((AssertionError, ValueError)):
            test_q8_0_dequant_bruteforce_all_codes()
        monkeypatch.undo()


# ------------------------------------------------------------------ router
def test_router_hand_example():
    """T = 1, H = 2, E = 4, k = 2: logits (1, 3, 3, -1) -> ids (1, 2) (equal logits by
    id), weights softmax(3, 3) = (1/2, 1/2); k = 3 adds expert 0 with weights
    e^3 : e^3 : e^1 normalized."""
    x = np.array([[1.0, 2.0]])
    Wr = np.array([[1.0, 0.0], [1.0, 1.0], [-1.0, 2.0], [1.0, -1.0]], np.float32)
    bits = W.f32_to_bf16_bits(Wr)
    ids, w, lg = O.router_topk(x, bits, 2)
    assert lg.tolist() == [[1.0, 3.0, 3.0, -1.0]]
    assert ids.tolist() == [[1, 2]] and np.allclose(w, [[0.5, 0.5]], rtol=0, atol=1e-15)
    ids, w, _ = O.router_topk(x, bits, 3)
    assert ids.tolist() == [[1, 2, 0]]
    z = math.exp(3) * 2 + math.exp(1)
    assert np.allclose(w, [[math.exp(3) / z, math.exp(3) / z, math.exp(1) / z]], rtol=1e-15, atol=0)


def test_router_against_sort_and_invariants():
    rng = np.random.default_rng(6)
    T, H, E, k = 20, 64, 40, 8
    x = rng.standard_normal((T, H))
    bits = W.draw_router(9, E, H)
    ids, w, lg = O.router_topk(x, bits, k)
    Wr = O.bf16_to_f64(bits)
    assert np.allclose(lg, x @ Wr.T, rtol=1e-14, atol=1e-14)
    for t in range(T):
        ref = np.argsort(-lg[t], kind="stable")[:k]
        assert ids[t].tolist() == ref.tolist()
        assert np.all(np.diff(lg[t, ids[t]]) <= 0) and len(set(ids[t].tolist())) == k
        assert abs(w[t].sum() - 1.0) < 1e-14 and np.all(np.diff(w[t]) <= 1e-16)
        # softmax over the selected logits == full softmax renormalized over them
        p = np.exp(lg[t] - lg[t].max())
        p /= p.sum()
        assert np.allclose(w[t], p[ids[t]] / p[ids[t]].sum(), rtol=1e-12)
    # k = E selects everything in descending order; weights are the full softmax
    ids_all, w_all, _ = O.router_topk(x[:2], bits, E)
    assert sorted(ids_all[0].tolist()) == list(range(E))


def test_router_bf16_weights_decode_and_negative_controls(monkeypatch):
    """The router matrix is read as bf16 (not fp16); a sign or tie-order slip fails."""
    x = np.array([[1.0, 2.0]])
    bits = np.array([[0x3F80, 0x0000], [0x4000, 0x0000], [0xC000, 0x4040]], np.uint16)  # 1, 2, (-2, 3)
    ids, _, lg = O.router_topk(x, bits, 2)
    assert lg.tolist() == [[1.0, 2.0, 4.0]] and ids.tolist() == [[2, 1]]
    as_fp16 = bits.view(np.float16).astype(np.float64)
    assert not np.allclose(x @ as_fp16.T, lg)
    def reversed_ties(x_, b_, k_):
        W_r = O.bf16_to_f64(b_)
        lg_ = x_ @ W_r.T
        ids_ = np.argsort(-lg_, axis=1)[:, ::-1][:, :k_][:, ::-1]
        return ids_.astype(np.int32), None, lg_
    monkeypatch.setattr(O, "router_topk", reversed_ties)
    with pytest.raises(AssertionError):
        test_router_hand_example()


# ------------------------------------------------------------------ shared expert
def _append_expert(lay, sh):
    """The routed layer with the shared expert's bytes appended as expert E."""
    def cat(a, b):
        return type(a)(np.concatenate([a.codes, b.codes]), np.concatenate([a.scales, b.scales]),
                       np.concatenate([a.gamma, b.gamma]))
    return W.Layer(cat(lay.gate, sh.gate), cat(lay.up, sh.up), cat(lay.down, sh.down), lay.E + 1, lay.H, lay.I)


def _shared_case(seed=41, E=6, H=32, I=64, T=7, k=3, down_fmt="nvfp4"):
    lay = W.draw_layer(seed, E=E, H=H, I=I, down_fmt=down_fmt)
    sh = W.draw_shared_expert(seed, H=H, I=I, down_fmt=down_fmt)
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[1, 0] = -1   # dropped routed slot: the shared expert still applies
    w = rng.random((T, k)).astype(np.float32)
    return lay, sh, ids, w


@pytest.mark.parametrize("down_fmt", ["nvfp4", "q8_0"])
def test_shared_expert_is_an_always_routed_expert_of_weight_one(down_fmt):
    """The reading, checked through the independent per-pair path: the shared expert gives
    the same result as the same bytes appended as expert E, routed by every token as one
    more slot with weight 1 (moe_pairwise dequantizes per pair; moe_with_shared groups)."""
    lay, sh, ids, w = _shared_case(down_fmt=down_fmt)
    T, k = ids.shape
    x = np.random.default_rng(3).standard_normal((T, lay.H))
    lay2 = _append_expert(lay, sh)
    ids2 = np.hstack([ids, np.full((T, 1), lay.E, np.int32)])
    w2 = np.hstack([w, np.ones((T, 1), np.float32)])
    ref = O.moe_pairwise(x, lay2, ids2, w2)
    got = O.moe_with_shared(x, lay, sh, ids, w)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    # the rows option selects rows of the same result
    rows = np.array([5, 1, 2])
    assert np.abs(O.moe_with_shared(x, lay, sh, ids, w, rows=rows) - ref[rows]).max() <= 1e-12 * np.abs(ref).max()
    # the W4A8 variant quantizes the shared expert's x and h rows like a routed pair's
    xb = W.draw_activations(3, T, lay.H)
    a = O.moe_w4a8(xb, lay2, ids2, w2)
    b = O.moe_w4a8_with_shared(xb, lay, sh, ids, w)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_shared_expert_identity_closed_form():
    """H = I = 32, the shared expert's gate, up and down are identity matrices (E2M1 code 2
    = 1.0 on the diagonal, E4M3 scale byte 0x38 = 1.0, global scales 1), the routed weights
    zero: out = SiLU(x) * x elementwise, i.e. x^2 / (1 + exp(-x))."""
    n = 32
    nib = np.zeros((n, n), np.uint8)
    nib[np.arange(n), np.arange(n)] = 2
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)[None]
    eye = W.Proj(codes, np.full((1, n, n // 16), 0x38, np.uint8), np.ones(1, np.float32))
    sh = W.Layer(eye, eye, eye, 1, n, n)
    lay = W.draw_layer(43, E=3, H=n, I=n)
    x = np.linspace(-6.0, 6.0, 2 * n).reshape(2, n)
    ids = np.array([[0, 2], [1, 1]], np.int32)
    w = np.zeros((2, 2), np.float32)
    out = O.moe_with_shared(x, lay, sh, ids, w)
    expect = x * x / (1.0 + np.exp(-x))
    assert np.allclose(out, expect, rtol=1e-14, atol=1e-300)


def test_shared_expert_negative_controls(monkeypatch):
    """Plausible mistakes in the shared term fail the pins above: weighting it by a router
    weight, adding it per routed slot, and dropping it for rows whose slots are dropped."""
    real = O.nvfp4_oracle.moe_with_shared

    def weighted_by_slot0(x, layer, shared, ids, w, rows=None, ffn=None):
        rows_ = np.arange(ids.shape[0]) if rows is None else np.asarray(rows)
        base = O.moe_grouped(x, layer, ids, w, rows=rows_, ffn=ffn)
        return base + w[rows_, :1].astype(np.float64) * O.expert_ffn(x[rows_], *O.nvfp4_oracle._expert(shared, 0))

    def once_per_slot(x, layer, shared, ids, w, rows=None, ffn=None):
        rows_ = np.arange(ids.shape[0]) if rows is None else np.asarray(rows)
        base = O.moe_grouped(x, layer, ids, w, rows=rows_, ffn=ffn)
        n = (ids[rows_] >= 0).sum(1, keepdims=True)
        return base + n * O.expert_ffn(x[rows_], *O.nvfp4_oracle._expert(shared, 0))

    def routed_only(x, layer, shared, ids, w, rows=None, ffn=None):
        return O.moe_grouped(x, layer, ids, w, rows=rows, ffn=ffn)

    for bad in (weighted_by_slot0, once_per_slot, routed_only):
        monkeypatch.setattr(O, "moe_with_shared", bad)
        with pytest.raises(AssertionError):
            test_shared_expert_is_an_always_routed_expert_of_weight_one("nvfp4")
        monkeypatch.undo()
    # routed_only also fails the closed form (zero routed weights leave only the shared term)
    monkeypatch.setattr(O, "moe_with_shared", routed_only)
    with pytest.raises(AssertionError):
        test_shared_expert_identity_closed_form()
    monkeypatch.undo()
    assert O.moe_with_shared is real


# ------------------------------------------------------------------ W4A4 (NVFP4 activations)
def _nvfp4_fixture_row():
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [6, 3, 1.5, 0.75, -0.25, 0.2, 5, -5]
    x[0, 15] = 0.3
    x[0, 16:19] = [0.3, -0.15, 0.075]
    return x


def test_quant_nvfp4_fixture():
    """The hand-worked row of tests/golden/quant_nvfp4_cases.txt."""
    line = [ln for ln in read_golden("quant_nvfp4_cases.txt") if ln.startswith("scales")][0]
    sc_hex, co_hex = line[len("scales"):].split("| codes")
    codes, scales, g = O.quant_rows_nvfp4(_nvfp4_fixture_row())
    assert [int(b, 16) for b in sc_hex.split()] == list(scales[0])
    assert [int(b, 16) for b in co_hex.split()] == list(codes[0])
    assert g[0] == np.float32(6.0) / np.float32(2688.0)


def _nearest_even(t, values):
    """Brute force over exact rationals: index of the value nearest to t, ties to the even
    index, values above the last to the last."""
    tf = Fraction(float(t))
    if tf >= Fraction(float(values[-1])):
        return len(values) - 1
    best = None
    for i, v in enumerate(values):
        d = abs(Fraction(float(v)) - tf)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_quant_nvfp4_bruteforce():
    """Random rows (with zeros, ties, tiny and saturating values): every scale byte is the
    E4M3 value nearest to fp32(blockmax / fp32(6 g)) with ties to even, and every code the
    E2M1 magnitude nearest to fp32(v / fp32(s g)) with ties to even (saturating at 6), found
    by exact rational brute force; the sign bit is that of v (-0.0 included)."""
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((6, 64)) * np.exp2(rng.integers(-30, 30, size=(6, 1)))).astype(np.float32)
    x[1, 16:32] = 0                       # a zero group
    x[0, 3] = np.float32(-0.0)            # signed zeros inside coded groups
    x[5, 40] = np.float32(-0.0)
    x[2, :] *= np.float32(1e-38)          # tiny values: scales underflow E4M3
    x[3, 5] = x[3].max() * 1.001 if x[3].max() > 0 else 1.0
    x[4, 0:16] = np.float32(0.25) * np.sign(x[4, 0:16] + 1e-30)  # ties on the E2M1 grid
    x[4, 16] = 6.0
    codes, scales, g = O.quant_rows_nvfp4(x)
    nib = O.unpack_codes(codes)
    e4 = [float(v) for v in O.E4M3_TABLE[:127]]
    e2 = [float(v) for v in O.E2M1_TABLE[:8]]
    for r in range(x.shape[0]):
        amax = np.float32(np.abs(x[r]).max())
        gr = np.float32(amax / np.float32(2688.0))
        assert g[r] == gr
        d6 = np.float32(np.float32(6.0) * gr)
        for b in range(4):
            blk = x[r, 16 * b:16 * b + 16]
            t = np.float32(np.float32(np.abs(blk).max()) / d6) if d6 > 0 else np.float32(0)
            assert scales[r, b] == _nearest_even(t, e4)
            sv = np.float32(O.E4M3_TABLE[scales[r, b]])
            den = np.float32(sv * gr)
            for k in range(16):
                c = int(nib[r, 16 * b + k])
                if den == 0:
                    assert c == 0
                    continue
                q = np.float32(blk[k] / den)
                assert (c & 7) == _nearest_even(abs(q), e2), (r, b, k, q)
                assert (c >> 3) == (1 if np.signbit(blk[k]) else 0)


def test_quant_nvfp4_signed_zero():
    """The code's sign bit is the input's: in a row of max 1.0 (g = 1/2688, scale 448, s g =
    1/6), 1.0 -> 6 (code 7), -0.0 -> code 8, +0.0 -> code 0, -1e-9 -> code 8 (magnitude 0)."""
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1], x[0, 2], x[0, 3] = 1.0, -0.0, 0.0, -1e-9
    codes, scales, g = O.quant_rows_nvfp4(x)
    assert scales[0, 0] == 0x7E and g[0] == np.float32(1.0) / np.float32(2688.0)
    assert list(O.unpack_codes(codes)[0, :4]) == [7, 8, 0, 8]


def test_quant_nvfp4_zero_and_nonfinite_rows():
    x = np.zeros((3, 32), np.float32)
    x[1, 3] = np.nan
    x[2, 7] = -np.inf
    codes, scales, g = O.quant_rows_nvfp4(x)
    assert not codes.any() and not scales.any()
    assert g[0] == 0 and np.isnan(g[1]) and g[2] == np.inf
    deq = O.dequant_rows_nvfp4(codes, scales, g)
    assert not deq[0].any() and np.isnan(deq[1]).all() and np.isnan(deq[2]).all()


def test_w4a4_ffn_composition_and_down_from_codes():
    """moe_w4a4 is the MoE over the dequantized NVFP4 activations with the hidden rows
    requantized the same way (composition of pinned pieces), and w4a4_down_from_codes on
    the oracle's own hidden codes reproduces it."""
    lay = W.draw_layer(15, E=5, H=64, I=48)
    xb = W.draw_activations(15, 9, 64)
    ids = W.draw_routing_zipf(15, 9, 5, 3)
    w = W.draw_router_weights(15, 9, 3)
    got = O.moe_w4a4(xb, lay, ids, w)
    xq = O.dequant_rows_nvfp4(*O.quant_rows_nvfp4(O.bf16_to_f64(xb).astype(np.float32)))
    ref = np.zeros_like(got)
    for t in range(9):
        for j in range(3):
            e = int(ids[t, j])
            g = O.linear(xq[t:t + 1], lay.gate.codes[e], lay.gate.scales[e], lay.gate.gamma[e])
            u = O.linear(xq[t:t + 1], lay.up.codes[e], lay.up.scales[e], lay.up.gamma[e])
            h = (O.silu(g) * u).astype(np.float32)
            hq = O.dequant_rows_nvfp4(*O.quant_rows_nvfp4(h))
            ref[t] += float(w[t, j]) * O.linear(hq, lay.down.codes[e], lay.down.scales[e], lay.down.gamma[e])[0]
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    pairs, hs = [], []
    for e, pe, h in O.w4a4_pair_hidden(xb, lay, ids):
        pairs.append(pe)
        hs.append(h)
    qc, qs, qg = O.quant_rows_nvfp4(np.concatenate(hs))
    again = O.w4a4_down_from_codes(qc, qs, qg, np.concatenate(pairs), lay, ids, w)
    assert np.abs(again - got).max() <= 1e-12 * np.abs(got).max()


def test_quant_nvfp4_negative_controls(monkeypatch):
    """Ties away from zero, a missing row scale, or a truncating E4M3 conversion fail a pin."""
    real = O.nvfp4_oracle._rne_table

    def ties_up(t, table):
        t = np.asarray(t, dtype=np.float64)
        hi = np.clip(np.searchsorted(table, t, side="left"), 0, len(table) - 1)
        lo = np.clip(hi - 1, 0, len(table) - 1)
        pick = np.where(t - table[lo] < table[hi] - t, lo, hi)
        return np.where(t >= table[-1], len(table) - 1, pick)

    def truncating(t, table):
        t = np.asarray(t, dtype=np.float64)
        idx = np.clip(np.searchsorted(table, t, side="right") - 1, 0, len(table) - 1)
        return np.where(t >= table[-1], len(table) - 1, idx)

    for bad in (ties_up, truncating):
        monkeypatch.setattr(O.nvfp4_oracle, "_rne_table", bad)
        with pytest.raises(AssertionError):
            test_quant_nvfp4_fixture()
        monkeypatch.undo()
    assert O.nvfp4_oracle._rne_table is real

    def no_row_scale(v32):
        codes, scales, g = real_q(v32)
        return real_q(np.asarray(v32, np.float32) / np.where(g > 0, g, 1)[:, None] / np.float32(2688.0))

    real_q = O.nvfp4_oracle.quant_rows_nvfp4
    monkeypatch.setattr(O, "quant_rows_nvfp4", no_row_scale)
    with pytest.raises(AssertionError):
        test_quant_nvfp4_fixture()
    monkeypatch.undo()
