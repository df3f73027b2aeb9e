"""GPU parity of the layer's shared expert ("Strata NVFP4" README, 0.1.39-nvfp4.2 entry:
the shared expert and its fused SwiGLU quantizer), through the C-ABI, against the float64
oracle (moe_with_shared) and against the same bytes appended as a routed expert."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, TOL, bf16_dev, bf16_out_to_f64, layer_dev, max_row_rel_l2

pytestmark = pytest.mark.gpu
nv = pytest.importorskip("nvfp4_quantized_moe_02_amd")


def _case(seed, E, H, I, T, k, down_fmt="nvfp4"):
    lay = W.draw_layer(seed, E=E, H=H, I=I, down_fmt=down_fmt)
    sh = W.draw_shared_expert(seed, H=H, I=I, down_fmt=down_fmt)
    xb = W.draw_activations(seed, T, H, outlier_frac=0.001)
    ids = W.draw_routing_zipf(seed, T, E, k, s=1.1)
    ids[min(3, T - 1), 0] = -1  # a dropped routed slot
    w = W.draw_router_weights(seed, T, k)
    return lay, sh, xb, ids, w


def _appended(dl, ds):
    """Device layer with the shared expert's bytes appended as expert E."""
    def cat(a, b):
        g = None if a.gamma is None else torch.cat([a.gamma, b.gamma])
        return type(a)(torch.cat([a.codes, b.codes]), torch.cat([a.scales, b.scales]), g)
    return nv.Layer(cat(dl.gate, ds.gate), cat(dl.up, ds.up), cat(dl.down, ds.down))


def _with_slot(ids, w, E):
    T = ids.shape[0]
    return (np.hstack([ids, np.full((T, 1), E, np.int32)]), np.hstack([w, np.ones((T, 1), np.float32)]))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_shared_matches_oracle(out_dtype):
    lay, sh, xb, ids, w = _case(61, E=8, H=512, I=256, T=300, k=4)
    y = nv.moe_prefill(bf16_dev(xb), layer_dev(lay), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                       out_dtype=out_dtype, shared=layer_dev(sh))
    got = y.cpu().numpy().astype(np.float64) if out_dtype == torch.float32 else bf16_out_to_f64(y)
    ref = O.moe_with_shared(O.bf16_to_f64(xb), lay, sh, ids, w)
    err = max_row_rel_l2(got, ref)
    print(f"prefill with shared expert ({out_dtype}): max row rel L2 {err:.3e}")
    assert err < (5e-4 if out_dtype == torch.float32 else TOL)


@pytest.mark.parametrize("act", ["bf16", "w4a8_f16", "w4a8"])
@pytest.mark.parametrize("down_fmt", ["nvfp4", "q8_0"])
def test_prefill_shared_equals_appended_expert_bitwise(act, down_fmt):
    """The shared call runs the same launches on the same routing as a call whose layer has
    the shared expert appended as expert E and whose tokens route to it with weight 1."""
    lay, sh, xb, ids, w = _case(63, E=6, H=512, I=256, T=280, k=4, down_fmt=down_fmt)
    dl, ds = layer_dev(lay), layer_dev(sh)
    x = bf16_dev(xb)
    a = nv.moe_prefill(x, dl, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), act=act,
                       out_dtype=torch.float32, shared=ds)
    ids2, w2 = _with_slot(ids, w, lay.E)
    b = nv.moe_prefill(x, _appended(dl, ds), torch.from_numpy(ids2).to(DEV), torch.from_numpy(w2).to(DEV), act=act,
                       out_dtype=torch.float32)
    assert torch.equal(a, b)


def test_prefill_shared_full_size_rows():
    """The 8192-token workload with a shared expert: >= 256 sampled rows against the oracle."""
    lay = W.draw_layer(W.config_seed(3))
    sh = W.draw_shared_expert(W.config_seed(3))
    wl = W.draw_workload(3)
    y = nv.moe_prefill(bf16_dev(wl.x), layer_dev(lay), torch.from_numpy(wl.ids).to(DEV),
                       torch.from_numpy(wl.w).to(DEV), shared=layer_dev(sh))
    rows = np.sort(np.random.default_rng(5).choice(wl.T, 256, replace=False))
    ref = O.moe_with_shared(O.bf16_to_f64(wl.x), lay, sh, wl.ids, wl.w, rows=rows)
    got = bf16_out_to_f64(y[torch.from_numpy(rows).to(DEV)])
    err = max_row_rel_l2(got, ref)
    print(f"prefill 8192 tokens with shared expert: max row rel L2 {err:.3e}")
    assert err < TOL


@pytest.mark.parametrize("T", [1, 4, 7])
def test_decode_shared_matches_oracle_and_appended(T):
    lay, sh, xb, ids, w = _case(65 + T, E=16, H=1024, I=512, T=T, k=8)
    dl, ds = layer_dev(lay), layer_dev(sh)
    x, ti, tw = bf16_dev(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    y = nv.moe_decode(x, dl, ti, tw, shared=ds)
    ref = O.moe_with_shared(O.bf16_to_f64(xb), lay, sh, ids, w)
    err = max_row_rel_l2(y.cpu().numpy(), ref)
    print(f"decode T={T} with shared expert: max row rel L2 {err:.3e}")
    assert err < 1e-5
    ids2, w2 = _with_slot(ids, w, lay.E)
    b = nv.moe_decode(x, _appended(dl, ds), torch.from_numpy(ids2).to(DEV), torch.from_numpy(w2).to(DEV))
    assert torch.equal(y, b)


def test_shared_id_equal_to_E_is_dropped():
    """A routed id equal to E is out of range for the routed experts: it is dropped (and
    counted), not sent to the shared expert, which only the library's own slot reaches."""
    lay, sh, xb, ids, w = _case(71, E=8, H=512, I=256, T=64, k=4)
    ids = ids.copy()
    ids[5, 2] = lay.E
    ids[9, 0] = lay.E
    dl, ds = layer_dev(lay), layer_dev(sh)
    x, ti, tw = bf16_dev(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    ws = torch.zeros(nv.prefill_workspace_size(64, 512, 256, 8, 4, shared=True), dtype=torch.uint8, device=DEV)
    y = nv.moe_prefill(x, dl, ti, tw, out_dtype=torch.float32, ws=ws, shared=ds)
    ref = O.moe_with_shared(O.bf16_to_f64(xb), lay, sh, ids, w)
    assert max_row_rel_l2(y.cpu().numpy(), ref) < 5e-4
    assert int(ws[:4].view(torch.int32).item()) == 3  # the -1 and the two ids equal to E
    xd, idd, wd = x[:4], ti[:4].contiguous(), tw[:4].contiguous()
    wsd = torch.zeros(nv.decode_workspace_size(4, 512, 256, 8, 4, shared=True), dtype=torch.uint8, device=DEV)
    yd = nv.moe_decode(xd, dl, idd, wd, ws=wsd, shared=ds)
    refd = O.moe_with_shared(O.bf16_to_f64(xb[:4]), lay, sh, ids[:4], w[:4])
    assert max_row_rel_l2(yd.cpu().numpy(), refd) < 1e-5


def test_shared_expert_hidden_beyond_fp16_range():
    """The shared expert's h far above the fp16 range (gate and up global scales x 2^12):
    the fused SwiGLU epilogue's per-block power-of-two scale keeps the fp16 h finite, and the
    output matches the float64 oracle."""
    lay, sh, xb, ids, w = _case(73, E=8, H=512, I=256, T=200, k=4)
    sh.gate.gamma = (sh.gate.gamma * 4096).astype(np.float32)
    sh.up.gamma = (sh.up.gamma * 4096).astype(np.float32)
    hmax = 0.0
    x64 = O.bf16_to_f64(xb)
    Wg, gg, Wu, gu, _, _ = O.nvfp4_oracle._expert(sh, 0)
    hmax = float(np.abs(O.silu((x64 @ Wg.T) * gg) * ((x64 @ Wu.T) * gu)).max())
    assert hmax > 65504 * 16, hmax
    y = nv.moe_prefill(bf16_dev(xb), layer_dev(lay), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV),
                       out_dtype=torch.float32, shared=layer_dev(sh))
    assert torch.isfinite(y).all()
    ref = O.moe_with_shared(x64, lay, sh, ids, w)
    err = max_row_rel_l2(y.cpu().numpy(), ref)
    print(f"shared expert with h up to {hmax:.3e}: max row rel L2 {err:.3e}")
    assert err < 5e-4


def test_shared_validation():
    lay, sh, xb, ids, w = _case(75, E=8, H=256, I=128, T=8, k=8)
    dl, ds = layer_dev(lay), layer_dev(sh)
    x, ti, tw = bf16_dev(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    # T * (topk + 1) = 72 decode pairs exceed the 64 the decode kernel holds
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.moe_decode(x, dl, ti, tw, shared=ds)
    assert ei.value.status == -2
    # a shared expert of another shape
    other = layer_dev(W.draw_shared_expert(75, H=256, I=256))
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.moe_prefill(x, dl, ti, tw, shared=other)
    assert ei.value.status == -1
    # a Q8_0 shared down beside an NVFP4 routed down
    q8 = layer_dev(W.draw_shared_expert(75, H=256, I=128, down_fmt="q8_0"))
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.moe_prefill(x, dl, ti, tw, shared=nv.Layer(ds.gate, ds.up, q8.down))
    assert ei.value.status == -2
