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
            p.scales[idx] = 0x7E00 if p.fmt == "q8_0" else 0x7F  # fp16 / E4M3 NaN
    return dl


def sparse_layer(seed, experts, E=W.EXPERTS, H=W.HIDDEN, I=W.INTER, down_fmt="nvfp4"):
    """A full-size device layer holding the seeded bytes of `experts` only; all other
    experts have NaN scales. Returns (device layer, host subset layer)."""
    import nvfp4_quantized_moe_02_amd as nv
    sub = W.draw_layer(seed, E=E, H=H, I=I, experts=experts, down_fmt=down_fmt)
    gam = W.draw_gammas(seed, E)

    def proj(name, N, K):
        p = getattr(sub, name)
        codes = torch.full((E, N, K // 2), 0x77, dtype=torch.uint8, device=DEV)
        scales = torch.full((E, N, K // 16), 0x7F, dtype=torch.uint8, device=DEV)
        ids = torch.from_numpy(sub.experts).to(DEV)
        codes[ids] = torch.from_numpy(p.codes).to(DEV)
        scales[ids] = torch.from_numpy(p.scales).to(DEV)
        return nv.Proj(codes, scales, torch.from_numpy(gam[name]).to(DEV))

    def q8_down():
        p = sub.down
        codes = torch.full((E, H, I), 0x11, dtype=torch.int8, device=DEV)
        scales = torch.full((E, H, I // 32), 0x7E00, dtype=torch.int16, device=DEV)  # fp16 NaN
        ids = torch.from_numpy(sub.experts).to(DEV)
        codes[ids] = torch.from_numpy(p.codes).to(DEV)
        scales[ids] = torch.from_numpy(p.scales.view(np.int16)).to(DEV)
        return nv.Q8Proj(codes, scales, None)

    down = q8_down() if down_fmt == "q8_0" else proj("down", H, I)
    dl = nv.Layer(proj("gate", I, H), proj("up", I, H), down)
    return dl, sub


def max_row_rel_l2(y, ref):
    return float(np.max(O.rel_l2_rows(y, ref)))


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def cover_rows(ids, E, n=1024, seed=0, tile=128):
    """Token rows whose pairs reach every routed expert, including, for each expert, the
    token of its first pair, of its last pair and of the first pair of its last (usually
    partial) row tile of `tile` sorted rows; then random rows up to n. Sorted."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    rng = np.random.default_rng(seed)
    rows = set()
    order = np.argsort(flat, kind="stable")
    sf = flat[order]
    starts = np.searchsorted(sf, np.arange(E), side="left")
    ends = np.searchsorted(sf, np.arange(E), side="right")
    for e in range(E):
        a, b = int(starts[e]), int(ends[e])
        if a == b:
            continue
        ps = order[a:b]
        for q in (ps[0], ps[-1], ps[((b - a - 1) // tile) * tile]):
            rows.add(int(q) // k)
    rest = np.setdiff1d(np.arange(T), np.fromiter(rows, dtype=np.int64))
    extra = max(0, n - len(rows))
    if extra and len(rest):
        rows.update(rng.choice(rest, size=min(extra, len(rest)), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def ws_region(ws, T, H, I, E, k, act, name, dtype):
    """A view of one intermediate region of a prefill workspace (after the stage that writes it)."""
    import nvfp4_quantized_moe_02_amd as nv
    off, nb = nv.prefill_workspace_region(T, H, I, E, k, act, name)
    return ws[off:off + nb].view(dtype)


def w4a8_strict(xb, lay, ids, w, rows, ws, got, act="w4a8_f16"):
    """The W4A8 checks, strict (the configuration text's "the oracle uses the same int8
    activations"), on the pairs of the given token rows after a prefill call on ws:
      (a) the staged x codes and scales equal the oracle's quantization bit for bit;
      (b) the GPU's fp32 h is within 1e-5 (per pair row, relative L2) of the oracle's;
      (c) the quantizer applied to the GPU's own fp32 h gives the GPU's int8 codes and
          scales bit for bit (same inputs, same rule);
      (d) the GPU's codes differ from the oracle's (the quantizer on the oracle's h) only by
          +-1, at elements whose h lies at a rounding tie within the (b) difference;
      (e) the oracle's down step and combine on the GPU's codes match the GPU's output
          rows within the 2e-3 bound, with no allowance.
    Returns a dict of the measured figures, including the end-to-end error against the
    oracle's own codes (reported, not bounded)."""
    T, k = ids.shape
    H, I, E = lay.H, lay.I, lay.E
    P = T * k
    reg = lambda name, dt: ws_region(ws, T, H, I, E, k, act, name, dt)  # noqa: E731
    rows = np.asarray(rows)
    # (a)
    xq = reg("x_staged", torch.int8).view(T, H)[torch.from_numpy(rows).to(ws.device)].cpu().numpy()
    xs = reg("x_rowscale", torch.float32)[torch.from_numpy(rows).to(ws.device)].cpu().numpy()
    rq, rs = O.quant_rows_i8(O.bf16_to_f64(xb[rows]).astype(np.float32))
    assert np.array_equal(xq, rq) and np.array_equal(xs.view(np.uint32), rs.view(np.uint32))
    # the pairs of the rows, their GPU sorted positions, GPU h, codes, scales
    inv = reg("pair_position", torch.int32).cpu().numpy()
    pairs, h_orc = [], []
    for e, pe, h, _ in O.w4a8_pair_hidden(xb, lay, ids, rows):
        pairs.append(rows[pe // k] * k + pe % k)
        h_orc.append(h)
    pairs = np.concatenate(pairs)
    h_orc = np.concatenate(h_orc)
    pos = torch.from_numpy(inv[pairs].astype(np.int64)).to(ws.device)
    assert (inv[pairs] >= 0).all()
    hg = reg("h", torch.float32).view(P, I)[pos].cpu().numpy()
    qg = reg("h_q", torch.int8).view(P, I)[pos].cpu().numpy()
    sg = reg("h_scale", torch.float32)[pos].cpu().numpy()
    # (b)
    h_err = float(np.max(O.rel_l2_rows(hg, h_orc)))
    assert h_err < 1e-5, h_err
    # (c)
    q_re, s_re = O.quant_rows_i8(hg)
    assert np.array_equal(q_re, qg) and np.array_equal(s_re.view(np.uint32), sg.view(np.uint32))
    # (d) the quantizer rounds the fp32 quotient h / s; a code can differ only where the
    #     oracle's quotient lies within the quotient difference of a .5 point, which (b)
    #     keeps below 127 * 1e-5 of a code step: flips are allowed only within 1e-3 of a tie
    q_o, s_o = O.quant_rows_i8(h_orc)
    d = qg.astype(np.int32) - q_o.astype(np.int32)
    assert np.abs(d).max(initial=0) <= 1
    with np.errstate(invalid="ignore", divide="ignore"):
        vq_o = (h_orc / np.where(s_o > 0, s_o, np.float32(1))[:, None]).astype(np.float32).astype(np.float64)
    flip = d != 0
    tie_dist = np.abs(vq_o - np.floor(vq_o) - 0.5)
    assert np.all(tie_dist[flip] <= 1e-3), float(tie_dist[flip].max())
    # (e)
    ref = O.w4a8_down_from_codes(qg, sg, pairs, lay, ids, w, rows=rows)
    err = max_row_rel_l2(got, ref)
    assert err < TOL, err
    e2e = max_row_rel_l2(got, O.w4a8_down_from_codes(q_o, s_o, pairs, lay, ids, w, rows=rows))
    return dict(err=err, err_vs_oracle_codes=e2e, h_err=h_err, flips=int(flip.sum()), codes=int(flip.size),
                near_ties=int((tie_dist < 1e-3).sum()))


def _nibbles(packed: np.ndarray) -> np.ndarray:
    """uint8 [R][K/2] -> codes [R][K] (low nibble first). Byte handling only."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def w4a4_strict(xb, lay, ids, w, rows, ws, got, act="w4a4"):
    """The W4A4 checks, strict as for W4A8, on the pairs of the given token rows after a
    prefill call on ws:
      (a) the staged x codes, block scales and row scales equal the oracle's NVFP4
          quantization bit for bit;
      (b) the GPU's fp32 h is within 1e-5 (per pair row, relative L2) of the oracle's;
      (c) the quantizer applied to the GPU's own fp32 h gives the GPU's codes, block scales
          and row scales bit for bit;
      (d) against the oracle's quantization of its own h: row scales within 1e-5; a block
          scale differs only where the two fp32 quotients blockmax / (6 g) agree to 1e-4
          (a rounding boundary between them); within blocks of equal scale a code differs
          only in magnitude by one step, where the two quotients v / (s g) agree to 1e-3
          (a tie between them), or as the sign of a zero; at most 1e-3 of the codes differ;
      (e) the oracle's down step and combine on the GPU's codes match the GPU's output rows
          within the 2e-3 bound.
    Returns the measured figures, including the end-to-end error against the oracle's own
    codes (reported, not bounded)."""
    T, k = ids.shape
    H, I, E = lay.H, lay.I, lay.E
    P = T * k
    reg = lambda name, dt: ws_region(ws, T, H, I, E, k, act, name, dt)  # noqa: E731
    rows = np.asarray(rows)
    rt = torch.from_numpy(rows).to(ws.device)
    # (a)
    xc = reg("x_staged", torch.uint8).view(T, H // 2)[rt].cpu().numpy()
    xs = reg("x_blockscale", torch.uint8).view(T, H // 16)[rt].cpu().numpy()
    xg = reg("x_rowscale", torch.float32)[rt].cpu().numpy()
    rc, rs, rg = O.quant_rows_nvfp4(O.bf16_to_f64(xb[rows]).astype(np.float32))
    assert np.array_equal(xc, rc) and np.array_equal(xs, rs) and np.array_equal(xg.view(np.uint32), rg.view(np.uint32))
    inv = reg("pair_position", torch.int32).cpu().numpy()
    pairs, h_orc = [], []
    for e, pe, h in O.w4a4_pair_hidden(xb, lay, ids, rows):
        pairs.append(rows[pe // k] * k + pe % k)
        h_orc.append(h)
    pairs = np.concatenate(pairs)
    h_orc = np.concatenate(h_orc)
    assert (inv[pairs] >= 0).all()
    pos = torch.from_numpy(inv[pairs].astype(np.int64)).to(ws.device)
    hg = reg("h", torch.float32).view(P, I)[pos].cpu().numpy()
    qc = reg("h_q", torch.uint8).view(P, I // 2)[pos].cpu().numpy()
    qs = reg("h_blockscale", torch.uint8).view(P, I // 16)[pos].cpu().numpy()
    qg = reg("h_scale", torch.float32)[pos].cpu().numpy()
    # (b)
    h_err = float(np.max(O.rel_l2_rows(hg, h_orc)))
    assert h_err < 1e-5, h_err
    # (c)
    c_re, s_re, g_re = O.quant_rows_nvfp4(hg)
    assert np.array_equal(c_re, qc) and np.array_equal(s_re, qs) and np.array_equal(g_re.view(np.uint32),
                                                                                      qg.view(np.uint32))
    # (d)
    oc, os_, og = O.quant_rows_nvfp4(h_orc)
    assert np.all(np.abs(qg.astype(np.float64) - og) <= 1e-5 * np.abs(og))
    G = I // 16
    bm_g = np.abs(hg).reshape(len(pairs), G, 16).max(-1)
    bm_o = np.abs(h_orc).reshape(len(pairs), G, 16).max(-1)
    t_g = (bm_g / (np.float32(6) * qg)[:, None]).astype(np.float32).astype(np.float64)
    t_o = (bm_o / (np.float32(6) * og)[:, None]).astype(np.float32).astype(np.float64)
    sflip = qs != os_
    assert np.all(np.abs(t_g - t_o)[sflip] <= 1e-4 * t_o[sflip])
    ng, no = _nibbles(qc), _nibbles(oc)
    same_blk = np.repeat(~sflip, 16, axis=1)
    mg, mo = ng & 7, no & 7
    cflip = (ng != no) & same_blk & ~((mg == 0) & (mo == 0))
    assert np.all(np.abs(mg.astype(np.int32) - mo.astype(np.int32))[cflip] == 1)
    assert np.all((ng >> 3)[cflip] == (no >> 3)[cflip])
    sv = np.repeat(np.asarray(O.E4M3_POS, dtype=np.float64)[os_], 16, axis=1)
    den_o = (sv.astype(np.float32) * og[:, None]).astype(np.float32).astype(np.float64)
    den_g = (np.repeat(np.asarray(O.E4M3_POS, dtype=np.float64)[qs], 16, axis=1).astype(np.float32)
             * qg[:, None]).astype(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        q_o = np.abs(h_orc / den_o)
        q_g = np.abs(hg.astype(np.float64) / den_g)
    assert np.all(np.abs(q_g - q_o)[cflip] <= 1e-3)
    nflip = int(sflip.sum()) * 16 + int(cflip.sum())
    assert nflip <= 1e-3 * ng.size, nflip
    # (e)
    ref = O.w4a4_down_from_codes(qc, qs, qg, pairs, lay, ids, w, rows=rows)
    err = max_row_rel_l2(got, ref)
    assert err < TOL, err
    e2e = max_row_rel_l2(got, O.w4a4_down_from_codes(oc, os_, og, pairs, lay, ids, w, rows=rows))
    return dict(err=err, err_vs_oracle_codes=e2e, h_err=h_err, scale_flips=int(sflip.sum()),
                code_flips=int(cflip.sum()), codes=int(ng.size))
