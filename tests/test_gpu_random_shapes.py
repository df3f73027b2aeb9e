"""Seeded random shapes within the documented limits, against the float64 oracle: the
prefill (bf16 activations, every launch variant the shape selects: 8 or 4 waves, scale
groups of 4 or 2 K-blocks) and the decode (one or two launches, every chunk-count variant up
to H = 2048, I = 1024), with Zipf routing plus duplicate and dropped ids; the W4A8 and W4A4
paths, the shared expert, the Q8_0 down projection and the router the same way. Each case
prints its shape and error, so a failure names the case."""
import numpy as np
import pytest
import torch

import nvfp4_quantized_moe_02_amd as nv
import oracle as O
import workloads as W
from gpu_util import DEV, TOL, bf16_dev, bf16_out_to_f64, layer_dev, max_row_rel_l2

pytestmark = pytest.mark.gpu


def _routing(rng, seed, T, E, k):
    """Zipf routing over E experts (k <= E distinct per token), then a few duplicates and
    ids outside [0, E), which the method drops."""
    kk = min(k, E)
    ids = np.full((T, k), -1, dtype=np.int32)
    ids[:, :kk] = W.draw_routing_zipf(seed, T, E, kk)
    for t in range(T):
        if kk < k:
            ids[t, kk:] = ids[t, 0]               # duplicates fill the slots past E
        if rng.random() < 0.05:
            ids[t, int(rng.integers(0, k))] = int(rng.choice([-1, E, E + 7]))
    w = rng.random((T, k)).astype(np.float32)
    return ids, w


def _prefill_case(seed):
    rng = np.random.default_rng(7000 + seed)
    H = int(rng.choice([256, 512, 768, 1024]))
    I = 128 * int(rng.integers(1, 7))            # 128 .. 768
    E = int(rng.integers(1, 40))
    k = int(rng.integers(1, 9))
    T = int(rng.integers(1, 420))
    return rng, H, I, E, k, T


def _decode_case(seed):
    rng = np.random.default_rng(9000 + seed)
    H = 32 * int(rng.integers(1, 65))            # 32 .. 2048
    I = 32 * int(rng.integers(1, 33))            # 32 .. 1024
    E = int(rng.integers(1, 80))
    T = int(rng.integers(1, 9))
    k = int(rng.integers(1, min(8, 64 // T) + 1))
    return rng, H, I, E, k, T


@pytest.mark.parametrize("seed", range(10))
def test_prefill_random_shape(seed):
    rng, H, I, E, k, T = _prefill_case(seed)
    print(f"prefill seed={seed} T={T} E={E} H={H} I={I} k={k}", flush=True)
    lay = W.draw_layer(500 + seed, E=E, H=H, I=I)
    xb = W.draw_activations(500 + seed, T, H)
    ids, w = _routing(rng, 500 + seed, T, E, k)
    ref = O.moe_grouped(O.bf16_to_f64(xb), lay, ids, w)
    dl = layer_dev(lay)
    x, ti, tw = bf16_dev(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    y32 = nv.moe_prefill(x, dl, ti, tw, out_dtype=torch.float32)
    yb = nv.moe_prefill(x, dl, ti, tw, out_dtype=torch.bfloat16)
    e32 = max_row_rel_l2(y32.cpu().numpy().astype(np.float64), ref)
    eb = max_row_rel_l2(bf16_out_to_f64(yb), ref)
    print(f"   max row rel L2: fp32 out {e32:.3e}, bf16 out {eb:.3e}")
    assert e32 < 1e-3  # the fp16 h rounding alone
    assert eb < TOL


@pytest.mark.parametrize("seed", range(10))
def test_decode_random_shape(seed):
    rng, H, I, E, k, T = _decode_case(seed)
    print(f"decode seed={seed} T={T} E={E} H={H} I={I} k={k}", flush=True)
    lay = W.draw_layer(600 + seed, E=E, H=H, I=I)
    xb = W.draw_activations(600 + seed, T, H)
    ids, w = _routing(rng, 600 + seed, T, E, k)
    ref = O.moe_grouped(O.bf16_to_f64(xb), lay, ids, w)
    dl = layer_dev(lay)
    y = nv.moe_decode(bf16_dev(xb), dl, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
    err = max_row_rel_l2(y.cpu().numpy().astype(np.float64), ref)
    print(f"   max row rel L2 {err:.3e}")
    assert err < 1e-5  # FP32 arithmetic throughout


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("act", ["w4a8_f16", "w4a8", "w4a4"])
def test_quantized_prefill_random_shape(act, seed):
    """The W4A8 (fp16 and int8 matrix cores) and W4A4 paths on random shapes, with their
    strict checks (the staged activation codes bit-exact, h, the requantized codes and the
    oracle's down step on the GPU's codes) on every token row; distinct experts per token."""
    from gpu_util import w4a4_strict, w4a8_strict
    rng, H, I, E, k, T = _prefill_case(20 + seed)
    k = min(k, E)
    print(f"{act} seed={seed} T={T} E={E} H={H} I={I} k={k}", flush=True)
    lay = W.draw_layer(700 + seed, E=E, H=H, I=I)
    xb = W.draw_activations(700 + seed, T, H, outlier_frac=0.001)
    ids = W.draw_routing_zipf(700 + seed, T, E, k)
    w = W.draw_router_weights(700 + seed, T, k)
    dl = layer_dev(lay)
    ws = torch.zeros(nv.prefill_workspace_size(T, H, I, E, k, act), dtype=torch.uint8, device=DEV)
    y = nv.moe_prefill(bf16_dev(xb), dl, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), act=act,
                       out_dtype=torch.float32, ws=ws)
    got = y.cpu().numpy().astype(np.float64)
    strict = w4a4_strict if act == "w4a4" else w4a8_strict
    stats = strict(xb, lay, ids, w, np.arange(T), ws, got, act=act)
    print(f"   {stats}")


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("variant", ["shared", "q8_down", "shared_q8_down"])
def test_layer_variants_random_shape(variant, seed):
    """The layer's shared expert and the Q8_0 down projection (and both), prefill and
    decode, on random shapes against the oracle."""
    down_fmt = "q8_0" if "q8" in variant else "nvfp4"
    with_shared = variant.startswith("shared")
    rng, H, I, E, k, T = _prefill_case(40 + seed)
    _, Hd, Id, Ed, kd, Td = _decode_case(40 + seed)
    kd = min(kd, 64 // Td - 1) if with_shared else kd  # the shared slot counts as one more pair
    print(f"{variant} seed={seed} prefill T={T} E={E} H={H} I={I} k={k}; decode T={Td} E={Ed} H={Hd} I={Id} "
          f"k={kd}", flush=True)
    for (tt, ee, hh, ii, kk, base) in ((T, E, H, I, k, 800), (Td, Ed, Hd, Id, kd, 900)):
        s = base + seed
        lay = W.draw_layer(s, E=ee, H=hh, I=ii, down_fmt=down_fmt)
        sh = W.draw_shared_expert(s, H=hh, I=ii, down_fmt=down_fmt) if with_shared else None
        xb = W.draw_activations(s, tt, hh)
        ids, w = _routing(np.random.default_rng(s), s, tt, ee, kk)
        x64 = O.bf16_to_f64(xb)
        ref = O.moe_with_shared(x64, lay, sh, ids, w) if with_shared else O.moe_grouped(x64, lay, ids, w)
        args = (bf16_dev(xb), layer_dev(lay), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV))
        shd = layer_dev(sh) if with_shared else None
        if base == 800:
            y = nv.moe_prefill(*args, out_dtype=torch.float32, shared=shd)
            bound = 1e-3  # the fp16 h (and a Q8_0 weight's one fp16 rounding)
        else:
            y = nv.moe_decode(*args, shared=shd)
            bound = 1e-5
        err = max_row_rel_l2(y.cpu().numpy().astype(np.float64), ref)
        print(f"   {'prefill' if base == 800 else 'decode'}: max row rel L2 {err:.3e}")
        assert err < bound


@pytest.mark.parametrize("seed", range(6))
def test_router_random_shape(seed):
    """The router (logits, top-k, softmax) on random shapes within its limits (H a multiple
    of 64, E a multiple of 32 up to 2048, k up to 64), bf16 and fp32 activations, with the
    checks of the router tests (logits within the fp32 accumulation bound, the selection and
    weights exact from those logits, the ids against the oracle's away from near-ties)."""
    from test_gpu_router import _run
    rng = np.random.default_rng(11000 + seed)
    H = 64 * int(rng.integers(1, 33))
    E = 32 * int(rng.integers(1, 65))
    k = int(rng.integers(1, min(64, E) + 1))
    T = int(rng.integers(1, 600))
    fp32 = bool(seed % 2)
    print(f"router seed={seed} T={T} E={E} H={H} k={k} x {'fp32' if fp32 else 'bf16'}", flush=True)
    wr = W.draw_router(1100 + seed, E=E, H=H)
    if fp32:
        x = (rng.standard_normal((T, H)) * np.exp(rng.uniform(-2, 2, (T, 1)))).astype(np.float32)
        ntie = _run(torch.from_numpy(x).to(DEV), x.astype(np.float64), wr, k)
    else:
        xb = W.draw_activations(1100 + seed, T, H)
        ntie = _run(bf16_dev(xb), O.bf16_to_f64(xb), wr, k)
    print(f"   {ntie} tokens with a near-tie at the k-th expert")
