"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and the
error measures. No arithmetic of the method lives here."""
import numpy as np
import torch

import oracle as O
import workloads as W

DEV = "cuda"
TOL = 2e-3  # max per-row relative L2 error against the float64 oracle


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)


def layer_dev(lay, fill_unused_nan=False, used=None):
    """Device copy of a workloads.Layer. With fill_unused_nan, experts outside `used`
    get NaN scale bytes, so any read of an unrouted expert poisons the output."""
    import nvfp4_quantized_moe_02_amd as nv
    dl = nv.Layer.from_numpy(lay, DEV)
    if fill_unused_nan:
        mask = np.ones(lay.E, dtype=bool)
        mask[np.asarray(sorted(set(int(e) for e in used if 0 <= e < lay.E)), dtype=np.int64)] = False
        idx = torch.from_numpy(np.nonzero(mask)[0]).to(DEV)
        for p in (dl.gate, dl.up, dl.down):
            p.scales[idx] = 0x7F
    return dl


def sparse_layer(seed, experts, E=W.EXPERTS, H=W.HIDDEN, I=W.INTER):
    """A full-size device layer holding the seeded bytes of `experts` only; all other
    experts have NaN scales. Returns (device layer, host subset layer)."""
    import nvfp4_quantized_moe_02_amd as nv
    sub = W.draw_layer(seed, E=E, H=H, I=I, experts=experts)
    gam = W.draw_gammas(seed, E)

    def proj(name, N, K):
        p = getattr(sub, name)
        codes = torch.full((E, N, K // 2), 0x77, dtype=torch.uint8, device=DEV)
        scales = torch.full((E, N, K // 16), 0x7F, dtype=torch.uint8, device=DEV)
        ids = torch.from_numpy(sub.experts).to(DEV)
        codes[ids] = torch.from_numpy(p.codes).to(DEV)
        scales[ids] = torch.from_numpy(p.scales).to(DEV)
        return nv.Proj(codes, scales, torch.from_numpy(gam[name]).to(DEV))

    dl = nv.Layer(proj("gate", I, H), proj("up", I, H), proj("down", H, I))
    return dl, sub


def max_row_rel_l2(y, ref):
    return float(np.max(O.rel_l2_rows(y, ref)))


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
