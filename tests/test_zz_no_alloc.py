"""The decode entry point that allocates nothing (nvfp4_moe_decode_noalloc, for callers
that cannot allocate) against the workspace entry point nvfp4_moe_decode, through the
C-ABI: same kernels, so the outputs must be identical bit for bit, on consecutive calls
that share the static scratch, the later ones smaller (fewer tokens, a smaller H, whose
grid is smaller), then the large shape again."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DEV, bf16_dev, layer_dev, sparse_layer

pytestmark = pytest.mark.gpu
nv = pytest.importorskip("nvfp4_quantized_moe_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(dl, xb, ids, w, out_dtype=torch.float32):
    x, ti, tw = bf16_dev(xb), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    ref = nv.moe_decode(x, dl, ti, tw, out_dtype=out_dtype)
    got = torch.full_like(ref, float("nan"))
    nv.moe_decode_noalloc(x, dl, ti, tw, got)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_decode_equals_workspace_decode():
    wl4 = W.draw_workload(2)   # 4 tokens, Zipf, the full layer shape
    wl1 = W.draw_workload(1)   # 1 token, uniform
    used = np.union1d(np.unique(wl4.ids), np.unique(wl1.ids))
    dl, _ = sparse_layer(wl4.seed, used)
    got, ref = _pair(dl, wl4.x, wl4.ids, wl4.w)
    assert torch.isfinite(ref).all() and torch.equal(got, ref), "4 tokens"
    got, ref = _pair(dl, wl1.x, wl1.ids, wl1.w)   # a smaller input on the same scratch
    assert torch.equal(got, ref), "1 token"
    # a smaller layer (H = 512: a grid of 64 blocks instead of 256), bf16 output
    lay = W.draw_layer(71, E=16, H=512, I=256)
    dls = layer_dev(lay)
    xb = W.draw_activations(71, 3, 512)
    ids = W.draw_routing_zipf(71, 3, 16, 8)
    w = W.draw_router_weights(71, 3, 8)
    got, ref = _pair(dls, xb, ids, w, out_dtype=torch.bfloat16)
    assert torch.equal(got, ref), "H = 512"
    # back to the large grid after the smaller one
    got, ref = _pair(dl, wl4.x, wl4.ids, wl4.w)
    assert torch.equal(got, ref), "4 tokens again"


def test_noalloc_rejects_what_does_not_fit():
    """More scratch than the array holds (h of 64 pairs x 8192 intermediate values is 2 MiB)
    is refused before anything is enqueued; so is a bad argument."""
    E, H, I = 2, 256, 8192
    lay = W.draw_layer(73, E=E, H=H, I=I)
    dl = layer_dev(lay)
    T, k = 8, 8
    x = bf16_dev(W.draw_activations(73, T, H))
    ids = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    w = torch.ones((T, k), dtype=torch.float32, device=DEV)
    out = torch.zeros((T, H), dtype=torch.float32, device=DEV)
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.moe_decode_noalloc(x, dl, ids, w, out)
    assert ei.value.status == -2
    # one token fits (8 pairs x 8192 x 4 bytes of h), but an fp16 output is not accepted
    with pytest.raises(nv.NVFP4Error) as ei:
        nv.moe_decode_noalloc(x[:1], dl, ids[:1], w[:1], torch.zeros((1, H), dtype=torch.float16, device=DEV))
    assert ei.value.status == -1
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0  # nothing was written
