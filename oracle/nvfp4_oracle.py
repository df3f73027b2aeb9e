"""CPU oracle for the NVFP4 routed-expert MoE projection.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library; both sides consume the same
seeded arrays from `workloads`.

Everything is plain numpy in float64. Dequantization is exact in float64 (an
E2M1 value has 2 significant bits, an E4M3 value 4, an FP32 global scale 24,
so a product has at most 30), so the dense float64 computation *is* the
definition of the method up to summation order. Library primitives used as
steps: numpy matrix products and numpy's float64->float32/float16 casts; torch
only for float32->bf16 rounding of outputs.

Sources (the pages, by title and section):
  [S-NVFP4]  "Strata NVFP4" README, section "How it differs from upstream
             Strata": NVFP4 keeps experts at 4.5 bits with calibrated scales;
             per-expert FP32 scales are kept and applied to each projection's
             output; W4A8 prompt path keeps 8-bit activations; a scale fold
             that left hidden activations in FP16 subnormals caused 2-12%
             expert error; the shared expert's fused SwiGLU quantizer.
  [TF-906]   TensorFold pull 906 (rank-local NVFP4 slice reader): plain E4M3
             scale bytes, input cuts preserve groups of 16, the FP32 tensor
             scale is unchanged by slicing; row and input partitions
             reassemble to the original bytes.
  [FP4-L]    #2727 "tools: add opt-in FP4-Local CSF checkpoint conversion",
             Validation list: expert tensors stack 512 experts; three-expert
             CUDA parity on relative output error.
  [S-RT]     "Strata NVFP4" README: the prompt path's BF16 projections (the
             router among them) take FP32-exact inputs. The routing rule itself
             is not on the pages; the reading taken: logits = x . Wr^T, the k
             largest (ties to the lower expert id) in descending order, router
             weights = softmax over those k logits.
  [S-MIX]    "Strata NVFP4" README, the re-quantized experts pack: in 27 of the
             48 layers the down projection is Q8_0 (more bytes, less error).
             The pages name the format but not its bytes; this oracle takes
             GGML's Q8_0 element rule: blocks of 32 int8 weights along the
             inputs, one fp16 scale d per block, weight = d * q (exact in
             float64: 8 + 11 significant bits).
Element formats are the public OCP Microscaling definitions that NVFP4 uses:
E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit, no inf/NaN) and
FP8 E4M3 "FN" (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no inf,
S.1111.111 is NaN, largest finite 448).

Readings where the pages are silent (each listed in the design notes):
  * element 2j of a row sits in the low nibble of byte j, 2j+1 in the high;
  * weights are [outputs][inputs]; the 16-groups run along the inputs;
  * the global scale multiplies the projection output; the gate's scale is
    applied before SiLU;
  * SwiGLU is SiLU(gate) * up with SiLU(z) = z / (1 + exp(-z)), no clamp;
  * router weights are used as given; duplicate ids are summed; ids outside
    [0, E) are dropped;
  * the shared expert is an NVFP4 SwiGLU expert of the routed experts' shape,
    applied to every token with weight 1 and added before the final rounding;
  * W4A4: activations quantized per row to NVFP4 with an FP32 row scale (the rule is
    stated beside quant_rows_nvfp4);
  * W4A8: per row s = fp32(absmax / 127) by an fp32 division, q = clamp(
    rint_even(fp32(x / s)), -127, 127), s = q = 0 for an all-zero row; the
    down projection's input h is quantized per (token, slot) row the same
    way, from h rounded to fp32; a row holding a NaN (an infinity) gets a NaN
    (+inf) scale and all-zero codes, so its non-finite value propagates.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

GROUP = 16


Q8_BLOCK = 32


# ----------------------------------------------------------------- element codecs
def e2m1_value(code):
    """E2M1 code (0..15) -> value. Bit fields s.ee.m; e == 0 is subnormal (m * 0.5),
    otherwise 2^(e-1) * (1 + m/2). Codes 0 and 8 are +0 and -0. [S-NVFP4]"""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return np.where(s == 1, -mag, mag)


def e4m3fn_value(byte):
    """FP8 E4M3 (FN variant) byte -> value. Bit fields s.eeee.mmm; e == 0 is
    subnormal (m * 2^-9), otherwise 2^(e-7) * (1 + m/8); e == 15 with m == 7 is
    NaN; there is no infinity. [TF-906] ("plain E4M3" scale bytes)"""
    b = np.asarray(byte, dtype=np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.exp2(e - 7.0) * (1.0 + m / 8.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


E2M1_TABLE = e2m1_value(np.arange(16))
E4M3_TABLE = e4m3fn_value(np.arange(256))


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """Packed bytes [..., K/2] -> codes [..., K]; element 2j = low nibble of byte j."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def pack_codes(nibbles: np.ndarray) -> np.ndarray:
    """Inverse of unpack_codes."""
    n = np.asarray(nibbles, dtype=np.uint8)
    if n.shape[-1] % 2:
        raise ValueError("odd number of codes")
    return (n[..., 0::2] & 0x0F) | ((n[..., 1::2] & 0x0F) << 4)


# ----------------------------------------------------------------- dequantization
def dequant(codes: np.ndarray, scales: np.ndarray, gamma: Optional[float] = None) -> np.ndarray:
    """W[n][k] = e2m1(code[n][k]) * e4m3(scale[n][k // 16]) [* gamma], float64, exact.
    [S-NVFP4] 4.5-bit experts; [TF-906] groups of 16 inputs and the FP32 tensor scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    K = codes.shape[-1] * 2
    if scales.shape[-1] * GROUP != K:
        raise ValueError("scale plane does not cover K in groups of 16")
    vals = E2M1_TABLE[unpack_codes(codes)]
    sc = E4M3_TABLE[scales]
    W = vals * np.repeat(sc, GROUP, axis=-1)
    if gamma is not None:
        W = W * float(np.float32(gamma))
    return W


def dequant_f32(codes, scales, gamma=None) -> np.ndarray:
    """One round-to-nearest-even rounding of the exact product to float32."""
    with np.errstate(invalid="ignore"):
        return dequant(codes, scales, gamma).astype(np.float32)


def bf16_bits(a32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch's conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def dequant_bf16(codes, scales, gamma=None) -> np.ndarray:
    """bf16 output: the exact product rounded to float32, then to bf16 (both
    nearest-even). Without gamma the product is exact in bf16 and both
    roundings are the identity."""
    return bf16_bits(dequant_f32(codes, scales, gamma))


def dequant_f16(codes, scales, gamma=None) -> np.ndarray:
    with np.errstate(invalid="ignore", over="ignore"):
        return dequant_f32(codes, scales, gamma).astype(np.float16)


# ----------------------------------------------------------------- linear algebra
def linear(x: np.ndarray, codes, scales, gamma) -> np.ndarray:
    """y[t][n] = gamma * sum_k x[t][k] * W[n][k]: rows of W are outputs, the
    global scale multiplies the output. [S-NVFP4] [TF-906]"""
    W = dequant(codes, scales)
    y = np.asarray(x, dtype=np.float64) @ W.T
    return y * float(np.float32(gamma))


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def dequant_q8_0(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q8_0 rows [S-MIX]: codes int8 [..][K], scales fp16 bit patterns (uint16)
    [..][K/32]; W[n][k] = fp16(scales[n][k // 32]) * codes[n][k], exact in float64."""
    q = np.asarray(codes, dtype=np.int8).astype(np.float64)
    d = np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64)
    K = q.shape[-1]
    assert K % Q8_BLOCK == 0 and d.shape[-1] * Q8_BLOCK == K
    return q * np.repeat(d, Q8_BLOCK, axis=-1)


def _dequant_proj(proj, s: int) -> np.ndarray:
    if getattr(proj, "fmt", "nvfp4") == "q8_0":
        return dequant_q8_0(proj.codes[s], proj.scales[s])
    return dequant(proj.codes[s], proj.scales[s])


def _expert(layer, e: int):
    s = layer.slot(e)
    return (
        _dequant_proj(layer.gate, s), float(layer.gate.gamma[s]),
        _dequant_proj(layer.up, s), float(layer.up.gamma[s]),
        _dequant_proj(layer.down, s), float(layer.down.gamma[s]),
    )


def expert_ffn(x: np.ndarray, Wg, gg, Wu, gu, Wd, gd) -> np.ndarray:
    """One routed expert on rows x [n][H]: y = gd * (SiLU(gg * x Wg^T) * (gu * x Wu^T)) Wd^T."""
    g = (x @ Wg.T) * gg
    u = (x @ Wu.T) * gu
    h = silu(g) * u
    return (h @ Wd.T) * gd


def moe_pairwise(x: np.ndarray, layer, ids: np.ndarray, w: np.ndarray,
                 rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """out[t] = sum_j w[t][j] * FFN_{ids[t][j]}(x[t]), one (token, slot) at a time,
    dequantizing the expert afresh for each pair. x is float64 [T][H]."""
    T, k = ids.shape
    rows = range(T) if rows is None else rows
    out = np.zeros((len(rows), layer.H), dtype=np.float64)
    for r, t in enumerate(rows):
        for j in range(k):
            e = int(ids[t, j])
            if e < 0 or e >= layer.E:
                continue
            y = expert_ffn(x[t:t + 1], *_expert(layer, e))[0]
            out[r] += float(w[t, j]) * y
    return out


def route(ids: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray]:
    """Counting sort of the pairs p = t*k + j by expert id.

    Returns offsets int32 [E+1] (exclusive prefix sum of per-expert counts,
    offsets[E] = number of valid pairs) and sorted_pairs int32 [T*k] listing
    the valid pairs ordered by (expert, p) ascending, padded with -1."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        if 0 <= e < E:
            counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_pairs = np.full(flat.shape[0], -1, dtype=np.int64)
    for p, e in enumerate(flat):
        if 0 <= e < E:
            sorted_pairs[cursor[e]] = p
            cursor[e] += 1
    return offsets.astype(np.int32), sorted_pairs.astype(np.int32)


def moe_grouped(x: np.ndarray, layer, ids: np.ndarray, w: np.ndarray,
                rows: Optional[Sequence[int]] = None, ffn=None) -> np.ndarray:
    """Same result as moe_pairwise, computed expert by expert: each expert is
    dequantized once and applied to all of its routed pairs."""
    T, k = ids.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    sel = ids[rows]
    offsets, sp = route(sel, layer.E)
    out = np.zeros((len(rows), layer.H), dtype=np.float64)
    ffn = expert_ffn if ffn is None else ffn
    for e in range(layer.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        pairs = sp[a:b]
        r_idx = pairs // k
        Y = ffn(x[rows[r_idx]], *_expert(layer, e))
        for i, p in enumerate(pairs):
            out[p // k] += float(w[rows[p // k], p % k]) * Y[i]
    return out


def moe_with_shared(x: np.ndarray, layer, shared, ids: np.ndarray, w: np.ndarray,
                    rows: Optional[Sequence[int]] = None, ffn=None) -> np.ndarray:
    """[S-NVFP4] (the shared expert) The routed sum plus the layer's shared expert:
    out[t] = sum_j w[t][j] * FFN_{ids[t][j]}(x[t]) + FFN_shared(x[t]). Reading (the pages
    give the shared expert no shape, format or weight): an NVFP4 SwiGLU expert of the
    routed experts' shape, applied to every token with weight 1 before the one final
    rounding. `shared` is a one-expert layer; ffn as in moe_grouped."""
    T = ids.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    ffn = expert_ffn if ffn is None else ffn
    out = moe_grouped(x, layer, ids, w, rows=rows, ffn=ffn)
    out += ffn(x[rows], *_expert(shared, 0))
    return out


# ----------------------------------------------------------------- router
def router_topk(x: np.ndarray, w_router_bf16_bits: np.ndarray, k: int):
    """[S-RT] x float64 [T][H] (exact values of the fp32 or bf16 inputs), Wr bf16 bits
    [E][H]. Returns (ids int32 [T][k], weights float64 [T][k], logits float64 [T][E]):
    logits = x Wr^T; ids = the k largest logits in descending order, equal logits
    ordered by expert id; weights = softmax of the k selected logits."""
    W_r = bf16_to_f64(np.asarray(w_router_bf16_bits, dtype=np.uint16))
    logits = np.asarray(x, dtype=np.float64) @ W_r.T
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    wts = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        ids[t] = order
        sel = logits[t, order]
        ex = np.exp(sel - sel[0])
        wts[t] = ex / ex.sum()
    return ids, wts, logits


# ----------------------------------------------------------------- W4A8
def quant_rows_i8(x32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int8: s = fp32(absmax / 127) (float32 division),
    q = clamp(round_half_even(fp32(x / s)), -127, 127); an all-zero row gives
    s = 0, q = 0. [S-NVFP4] W4A8 prompt path with 8-bit activations.

    Non-finite rows (a reading; the pages are silent): if a row holds a NaN, its
    absmax and so its scale are NaN; else if it holds an infinity, its scale is +inf.
    Either way every code of the row is 0, so the dequantized row q * s is NaN
    everywhere (0 * NaN, 0 * inf) and the non-finite value propagates to every output
    that row touches, as a NaN or infinite activation does in float64."""
    x32 = np.asarray(x32, dtype=np.float32)
    a = np.abs(x32)
    has_nan = np.isnan(a).any(axis=-1)
    absmax = np.where(has_nan, np.float32(np.nan), np.max(np.where(np.isnan(a), 0, a), axis=-1))
    absmax = absmax.astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        s = (absmax / np.float32(127.0)).astype(np.float32)
    finite = np.isfinite(s) & (s > 0)
    safe = np.where(finite, s, np.float32(1.0)).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint((np.where(finite[..., None], x32, 0) / safe[..., None]).astype(np.float32))
    q = np.clip(r, -127, 127)
    q = np.where(finite[..., None], q, 0).astype(np.int8)
    return q, s


def w4a8_hidden(xq: np.ndarray, Wg, gg, Wu, gu) -> np.ndarray:
    """The W4A8 expert's hidden rows on already-dequantized int8 activations
    x_hat = q * s (float64): h = SiLU(gg * x Wg^T) * (gu * x Wu^T), rounded to fp32
    (the value the down projection's int8 quantization starts from)."""
    g = (xq @ Wg.T) * gg
    u = (xq @ Wu.T) * gu
    return (silu(g) * u).astype(np.float32)


def w4a8_expert_ffn(xq: np.ndarray, Wg, gg, Wu, gu, Wd, gd) -> np.ndarray:
    """Expert FFN on already-dequantized int8 activations: h (fp32) is quantized per
    row to int8, and the down projection consumes h_hat = q_h * s_h."""
    qh, sh = quant_rows_i8(w4a8_hidden(xq, Wg, gg, Wu, gu))
    hh = qh.astype(np.float64) * sh.astype(np.float64)[:, None]
    return (hh @ Wd.T) * gd


def w4a8_activations(x_bf16_bits: np.ndarray) -> np.ndarray:
    """x (bf16) -> per-row int8 quantization -> x_hat = q * s in float64."""
    x32 = bf16_to_f64(x_bf16_bits).astype(np.float32)
    q, s = quant_rows_i8(x32)
    return q.astype(np.float64) * s.astype(np.float64)[:, None]


def moe_w4a8(x_bf16_bits: np.ndarray, layer, ids, w, rows=None) -> np.ndarray:
    """W4A8 MoE: both expert GEMMs take per-row int8 activations."""
    xh = w4a8_activations(x_bf16_bits)
    return moe_grouped(xh, layer, ids, w, rows=rows, ffn=w4a8_expert_ffn)


def moe_w4a8_with_shared(x_bf16_bits: np.ndarray, layer, shared, ids, w, rows=None) -> np.ndarray:
    """W4A8 MoE with the shared expert (moe_with_shared's reading): the shared expert's
    GEMMs take the same per-row int8 activations as the routed experts' (x per token, h
    per (token, shared) row)."""
    xh = w4a8_activations(x_bf16_bits)
    return moe_with_shared(xh, layer, shared, ids, w, rows=rows, ffn=w4a8_expert_ffn)


def w4a8_pair_hidden(x_bf16_bits: np.ndarray, layer, ids, rows=None):
    """For the routed pairs of the given token rows, expert by expert in route()
    order: (expert id, sorted pair indices into ids[rows], fp32 hidden rows h, their
    int8 scales s), i.e. the inputs of every requantization decision moe_w4a8 takes."""
    xh = w4a8_activations(x_bf16_bits)
    T, k = ids.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    offsets, sp = route(ids[rows], layer.E)
    out = []
    for e in range(layer.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        pairs = sp[a:b]
        Wg, gg, Wu, gu, _, _ = _expert(layer, e)
        h = w4a8_hidden(xh[rows[pairs // k]], Wg, gg, Wu, gu)
        _, s = quant_rows_i8(h)
        out.append((e, pairs, h, s))
    return out


def w4a8_down_from_codes(qh: np.ndarray, sh: np.ndarray, pairs: np.ndarray, layer, ids: np.ndarray,
                         w: np.ndarray, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The W4A8 down projection and combine on given int8 hidden rows: for each listed
    pair p = t*k + j (row i of qh, sh), out[t] += w[t][j] * gamma_d * (qh[i] * sh[i]) .
    Wd_e^T with e = ids[t][j]. This is the last step of moe_w4a8 with the hidden codes
    supplied by the caller (the configuration text's "the oracle uses the same int8
    activations" read literally for the requantized h). Returns float64 [T][H], or only the
    given token rows (every listed pair must belong to one of them)."""
    T, k = ids.shape
    pairs = np.asarray(pairs, dtype=np.int64)
    hh = np.asarray(qh, dtype=np.int8).astype(np.float64) * np.asarray(sh, dtype=np.float32).astype(np.float64)[:, None]
    row_of = {t: t for t in range(T)} if rows is None else {int(t): i for i, t in enumerate(rows)}
    out = np.zeros((len(row_of), layer.H), dtype=np.float64)
    ex = ids.reshape(-1)[pairs]
    for e in np.unique(ex):
        if e < 0 or e >= layer.E:
            continue
        sel = np.nonzero(ex == e)[0]
        _, _, _, _, Wd, gd = _expert(layer, int(e))
        Y = (hh[sel] @ Wd.T) * gd
        for i, r in enumerate(sel):
            p = int(pairs[r])
            out[row_of[p // k]] += float(w[p // k, p % k]) * Y[i]
    return out


# ----------------------------------------------------------------- W4A4
# [S-NVFP4] W4A8 bullet: llama.cpp builds the NVFP4 prompt path as FP4 x FP4, i.e. the
# activations are quantized to NVFP4 too. The pages give no activation quantization rule;
# the reading taken (r9): per row an FP32 scale g = fp32(absmax / 2688) (2688 = 6 * 448, so
# the largest block scale is 448), per 16 inputs an E4M3 scale s = E4M3_RNE(fp32(blockmax /
# fp32(6 g))) (saturating at 448), and per input the E2M1 code nearest to fp32(v / fp32(s g))
# with ties to the even code (saturating at 6), its sign bit the sign bit of v (so -0.0 and
# negative values that round to zero give the negative-zero code). A zero row has
# g = 0 and all codes and scales 0; a zero or underflowed block scale gives zero codes. A row
# holding a NaN gets g = NaN, else one holding an infinity g = +inf, with zero codes and
# scales, so the dequantized row (code * s * g) is NaN and propagates.

E4M3_POS = E4M3_TABLE[:127]          # the finite non-negative E4M3 values, codes 0..126, ascending
E2M1_POS = E2M1_TABLE[:8]            # 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7)


def _rne_table(t: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to each t >= 0 (table ascending, index parity =
    mantissa parity), ties to the even index; values above the last entry take the last."""
    t = np.asarray(t, dtype=np.float64)
    hi = np.clip(np.searchsorted(table, t, side="left"), 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dlo, dhi = t - table[lo], table[hi] - t
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return np.where(t >= table[-1], len(table) - 1, pick)


def quant_rows_nvfp4(v32: np.ndarray):
    """Rows of fp32 values [R][K] (K % 16 == 0) -> (codes uint8 [R][K/2], two per byte, low
    nibble first; scales uint8 [R][K/16] E4M3; g float32 [R]) by the r9 rule above. Every
    quotient is one fp32 operation on fp32 operands; the two roundings to the nearest table
    value are done on exact float64 copies of those quotients."""
    v = np.asarray(v32, dtype=np.float32)
    R, K = v.shape
    G = K // GROUP
    a = np.abs(v)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore", under="ignore"):
        nan_row = np.isnan(v).any(axis=1)
        amax = a.max(axis=1) if K else np.zeros(R, np.float32)
        inf_row = ~nan_row & np.isinf(amax)
        g = np.where(nan_row, np.float32(np.nan),
                     np.where(inf_row, np.float32(np.inf), amax / np.float32(2688.0))).astype(np.float32)
        live = ~nan_row & ~inf_row & (amax > 0)          # rows that get codes
        d6 = (np.float32(6.0) * g).astype(np.float32)
        live &= d6 > 0
        # block scales: t = blockmax / (6 g) in fp32, then the nearest E4M3 value
        bmax = a.reshape(R, G, GROUP).max(axis=2)
        t = (bmax / np.where(live, d6, np.float32(1))[:, None]).astype(np.float32)
        si = np.where(live[:, None], _rne_table(t.astype(np.float64), E4M3_POS), 0).astype(np.uint8)
        # codes: v / (s g) in fp32 (s g rounded to fp32 first), then the nearest E2M1 value
        den = (E4M3_POS[si].astype(np.float32) * g[:, None]).astype(np.float32)
        coded = live[:, None] & (den > 0)
        q = (v.reshape(R, G, GROUP) / np.where(coded, den, np.float32(1))[:, :, None]).astype(np.float32)
        mag = _rne_table(np.abs(q).astype(np.float64), E2M1_POS).astype(np.uint8)
        nib = np.where(coded[:, :, None], mag | np.where(np.signbit(v.reshape(R, G, GROUP)), 8, 0).astype(np.uint8), 0)
    return pack_codes(nib.reshape(R, K).astype(np.uint8)), si, g


def dequant_rows_nvfp4(codes: np.ndarray, scales: np.ndarray, g: np.ndarray) -> np.ndarray:
    """code * scale * g in float64 (exact: 2 + 4 + 24 significant bits); a NaN or infinite
    row scale with zero codes gives NaN (0 * inf)."""
    with np.errstate(invalid="ignore"):
        return dequant(codes, scales) * np.asarray(g, dtype=np.float32).astype(np.float64)[:, None]


def w4a4_activations(x_bf16_bits: np.ndarray) -> np.ndarray:
    """x (bf16) -> per-row NVFP4 quantization -> dequantized x in float64."""
    return dequant_rows_nvfp4(*quant_rows_nvfp4(bf16_to_f64(x_bf16_bits).astype(np.float32)))


def w4a4_expert_ffn(xq: np.ndarray, Wg, gg, Wu, gu, Wd, gd) -> np.ndarray:
    """Expert FFN on already-dequantized NVFP4 activations: h (fp32) is quantized per row
    to NVFP4 by the same rule, and the down projection consumes the dequantized h."""
    h = w4a8_hidden(xq, Wg, gg, Wu, gu)
    return (dequant_rows_nvfp4(*quant_rows_nvfp4(h)) @ Wd.T) * gd


def moe_w4a4(x_bf16_bits: np.ndarray, layer, ids, w, rows=None) -> np.ndarray:
    """W4A4 MoE: both expert GEMMs take per-row NVFP4 activations (reading r9)."""
    return moe_grouped(w4a4_activations(x_bf16_bits), layer, ids, w, rows=rows, ffn=w4a4_expert_ffn)


def w4a4_pair_hidden(x_bf16_bits: np.ndarray, layer, ids, rows=None):
    """For the routed pairs of the given token rows, expert by expert in route() order:
    (expert id, sorted pair indices into ids[rows], fp32 hidden rows h)."""
    xh = w4a4_activations(x_bf16_bits)
    T, k = ids.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    offsets, sp = route(ids[rows], layer.E)
    out = []
    for e in range(layer.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        pairs = sp[a:b]
        Wg, gg, Wu, gu, _, _ = _expert(layer, e)
        out.append((e, pairs, w4a8_hidden(xh[rows[pairs // k]], Wg, gg, Wu, gu)))
    return out


def w4a4_down_from_codes(qc: np.ndarray, qs: np.ndarray, qg: np.ndarray, pairs: np.ndarray, layer,
                         ids: np.ndarray, w: np.ndarray, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The W4A4 down projection and combine on given NVFP4 hidden rows (codes, scales, row
    scales; row i belongs to pair pairs[i] = t*k + j): out[t] += w[t][j] * gamma_d * h_hat .
    Wd_e^T. Returns float64 [T][H], or only the given token rows."""
    T, k = ids.shape
    pairs = np.asarray(pairs, dtype=np.int64)
    hh = dequant_rows_nvfp4(qc, qs, qg)
    row_of = {t: t for t in range(T)} if rows is None else {int(t): i for i, t in enumerate(rows)}
    out = np.zeros((len(row_of), layer.H), dtype=np.float64)
    ex = ids.reshape(-1)[pairs]
    for e in np.unique(ex):
        if e < 0 or e >= layer.E:
            continue
        sel = np.nonzero(ex == e)[0]
        _, _, _, _, Wd, gd = _expert(layer, int(e))
        Y = (hh[sel] @ Wd.T) * gd
        for i, r in enumerate(sel):
            p = int(pairs[r])
            out[row_of[p // k]] += float(w[p // k, p % k]) * Y[i]
    return out


# ----------------------------------------------------------------- comparison
def rel_l2_rows(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row relative L2 error ||y - ref|| / ||ref|| (rows with ||ref|| = 0
    report ||y||)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((y - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(ref ** 2, axis=-1))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)

