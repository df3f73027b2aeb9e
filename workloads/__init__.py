"""Seeded synthetic inputs for the NVFP4 routed-expert MoE projection.

This module only draws inputs. It holds none of the method's arithmetic: no
E2M1/E4M3 decoding, no products, no SwiGLU, no combine. Both the CPU oracle and
the GPU path consume exactly the arrays produced here.

Shapes follow the model the pages describe: 512 routed experts per layer
(#2727 "tools: add opt-in FP4-Local CSF checkpoint conversion", Validation list:
144 NVFP4 expert tensors with 512 experts each, 48 layers), each expert holding
three NVFP4 projections (gate, up, down). Hidden size 2048 and expert
intermediate size 768 are the layer shape used throughout.

Array conventions (all numpy, C-contiguous):
  codes  uint8 [E][N][K/2]   two E2M1 codes per byte, element 2j in the low nibble
  scales uint8 [E][N][K/16]  one FP8 E4M3 byte per 16 consecutive inputs
  gamma  float32 [E]         one FP32 global scale per expert tensor
  x      uint16 [T][H]       bf16 bit patterns (fp32 for the single-expert case)
  ids    int32 [T][k]        routed expert ids
  w      float32 [T][k]      router weights

Recipe (per config index c, seed = 20261203 + c, numpy PCG64):
  * code bytes: uniform over 0..255 (every byte is a valid pair of codes);
  * scale bytes: uniform over the 65 codes 0x18..0x58, i.e. the positive
    finite E4M3 values 2^-4 .. 2^4;
  * gamma: fp32(2^u / 2688), u ~ U[-1, 1], per (expert, projection); the
    single-expert case keeps fp32(1/2688) exactly (2688 = 6 * 448, the product
    of the largest E2M1 and E4M3 magnitudes);
  * activations: N(0, 1) drawn in fp64, rounded to fp32, optional outliers
    (a fraction of positions, chosen without replacement, multiplied by 20),
    then rounded to bf16 (round to nearest even, by torch's conversion);
  * routing: k distinct experts per token, either uniform without replacement
    or Zipf(s) over a seeded random permutation of expert ids, drawn by
    Gumbel-top-k (equivalent to sequential weighted sampling without
    replacement);
  * router weights: softmax of k i.i.d. N(0, 1) logits, in fp32.

Q8_0 down projections (the "Strata NVFP4" README's mixed pack: an 8-bit down
projection in selected layers; the format is GGML's Q8_0, blocks of 32 int8 weights
along the inputs with one fp16 scale each):
  codes  int8   [E][N][K]      one weight per byte
  scales uint16 [E][N][K/32]   fp16 bit patterns, scale b covers inputs 32b .. 32b+31
  gamma  float32 [E]           all 1.0 (the format has no tensor scale)
Recipe: code bytes uniform over all 256 values; scale = fp16(2^v / 8192) with
v ~ U[-1, 1] per block (always a normal fp16 value), so weights are of the same
order as the NVFP4 ones.

Router (the step before the MoE: "Strata NVFP4" README, the prompt path's BF16
projections, the router among them, fed FP32-exact inputs):
  w_router uint16 [E][H]  bf16 bit patterns, N(0, 1) / sqrt(H) rounded to bf16, plus a
                          per-expert bias row direction so that expert popularity is
                          uneven (expert e's row gets + b_e * u, u a shared unit vector,
                          b_e ~ N(0, 0.5)).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Iterable, Optional

import numpy as np
import torch

BASE_SEED = 20261203
HIDDEN = 2048
INTER = 768
EXPERTS = 512
TOPK = 8
GROUP = 16

PROJ_TAG = {"gate": 1, "up": 2, "down": 3, "down_q8": 4, "router": 5}
Q8_BLOCK = 32
_TAG_X, _TAG_IDS, _TAG_W, _TAG_GAMMA, _TAG_OUTLIER, _TAG_PERM = 11, 12, 13, 14, 15, 16
_TAG_SHARED = 17


def config_seed(index: int) -> int:
    return BASE_SEED + int(index)


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tags])))


@dataclass
class Proj:
    """One NVFP4 projection of E experts: rows = outputs (N), inputs = K."""
    codes: np.ndarray   # uint8 [E][N][K/2]
    scales: np.ndarray  # uint8 [E][N][K/16]
    gamma: np.ndarray   # float32 [E]

    @property
    def N(self) -> int:
        return int(self.codes.shape[1])

    @property
    def K(self) -> int:
        return int(self.codes.shape[2]) * 2


@dataclass
class Q8Proj:
    """One Q8_0 projection of E experts: rows = outputs (N), inputs = K."""
    codes: np.ndarray   # int8 [E][N][K]
    scales: np.ndarray  # uint16 (fp16 bits) [E][N][K/32]
    gamma: np.ndarray   # float32 [E]
    fmt = "q8_0"

    @property
    def N(self) -> int:
        return int(self.codes.shape[1])

    @property
    def K(self) -> int:
        return int(self.codes.shape[2])


Proj.fmt = "nvfp4"


@dataclass
class Layer:
    gate: Proj
    up: Proj
    down: "Proj | Q8Proj"
    E: int
    H: int
    I: int
    experts: Optional[np.ndarray] = None  # ids present, when only a subset was drawn
    index: Dict[int, int] = field(default_factory=dict)

    def slot(self, e: int) -> int:
        """Position of expert id e in the arrays (identity for a full layer)."""
        if self.experts is None:
            return int(e)
        return self.index[int(e)]


def draw_proj_expert(seed: int, proj: str, e: int, N: int, K: int):
    """Codes and scale bytes of one expert's projection, from its own stream."""
    g = _rng(seed, PROJ_TAG[proj], int(e))
    codes = np.frombuffer(g.bytes(N * K // 2), dtype=np.uint8).reshape(N, K // 2)
    scales = g.integers(0x18, 0x59, size=(N, K // GROUP), dtype=np.uint8)
    return codes, scales


def draw_q8_expert(seed: int, e: int, N: int, K: int):
    """Q8_0 code bytes (int8) and fp16 scale bits of one expert's down projection."""
    g = _rng(seed, PROJ_TAG["down_q8"], int(e))
    codes = np.frombuffer(g.bytes(N * K), dtype=np.int8).reshape(N, K).copy()
    v = g.uniform(-1.0, 1.0, size=(N, K // Q8_BLOCK))
    scales = (np.exp2(v) / 8192.0).astype(np.float16).view(np.uint16)
    return codes, scales


def draw_router(seed: int, E: int = EXPERTS, H: int = HIDDEN) -> np.ndarray:
    """bf16 bits [E][H] of a router matrix (see the module recipe)."""
    g = _rng(seed, PROJ_TAG["router"])
    w = g.standard_normal((E, H)) / np.sqrt(H)
    u = g.standard_normal(H)
    u /= np.linalg.norm(u)
    w += g.normal(0.0, 0.5, size=(E, 1)) * u[None, :]
    return f32_to_bf16_bits(w.astype(np.float32))


def draw_gammas(seed: int, E: int) -> Dict[str, np.ndarray]:
    g = _rng(seed, _TAG_GAMMA)
    u = g.uniform(-1.0, 1.0, size=(3, E))
    out = {}
    for i, p in enumerate(("gate", "up", "down")):
        out[p] = (np.exp2(u[i]) / 2688.0).astype(np.float32)
    return out


def draw_layer(seed: int, E: int = EXPERTS, H: int = HIDDEN, I: int = INTER,
               experts: Optional[Iterable[int]] = None, down_fmt: str = "nvfp4") -> Layer:
    """A full layer (experts=None) or only the listed experts (same bytes). down_fmt
    "q8_0" draws the down projection in Q8_0 instead of NVFP4."""
    gam = draw_gammas(seed, E)
    ids = np.arange(E) if experts is None else np.array(sorted(set(int(e) for e in experts)), dtype=np.int64)
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    projs = {}
    if down_fmt == "q8_0":
        codes = np.empty((len(ids), H, I), dtype=np.int8)
        scales = np.empty((len(ids), H, I // Q8_BLOCK), dtype=np.uint16)
        for s, e in enumerate(ids):
            codes[s], scales[s] = draw_q8_expert(seed, int(e), H, I)
        projs["down"] = Q8Proj(codes, scales, np.ones(len(ids), dtype=np.float32))
        del shapes["down"]
    elif down_fmt != "nvfp4":
        raise ValueError(down_fmt)
    for p, (N, K) in shapes.items():
        codes = np.empty((len(ids), N, K // 2), dtype=np.uint8)
        scales = np.empty((len(ids), N, K // GROUP), dtype=np.uint8)
        for s, e in enumerate(ids):
            codes[s], scales[s] = draw_proj_expert(seed, p, int(e), N, K)
        projs[p] = Proj(codes, scales, gam[p][ids].copy())
    lay = Layer(projs["gate"], projs["up"], projs["down"], E, H, I)
    if experts is not None:
        lay.experts = ids
        lay.index = {int(e): i for i, e in enumerate(ids)}
    return lay


def draw_shared_expert(seed: int, H: int = HIDDEN, I: int = INTER, down_fmt: str = "nvfp4") -> Layer:
    """The layer's shared expert: a one-expert layer of the routed experts' shape, drawn from
    streams of its own (the routed layer of the same seed is unrelated to it)."""
    return draw_layer(int(_rng(seed, _TAG_SHARED).integers(1 << 31)), E=1, H=H, I=I, down_fmt=down_fmt)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw_activations(seed: int, T: int, H: int = HIDDEN, outlier_frac: float = 0.0) -> np.ndarray:
    """bf16 bit patterns [T][H]."""
    g = _rng(seed, _TAG_X)
    x = g.standard_normal((T, H)).astype(np.float32)
    if outlier_frac > 0:
        n_out = int(round(outlier_frac * T * H))
        go = _rng(seed, _TAG_OUTLIER)
        pos = go.choice(T * H, size=n_out, replace=False)
        flat = x.reshape(-1)
        flat[pos] = flat[pos] * np.float32(20.0)
    return f32_to_bf16_bits(x)


def draw_routing_uniform(seed: int, T: int, E: int = EXPERTS, k: int = TOPK) -> np.ndarray:
    g = _rng(seed, _TAG_IDS)
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = g.choice(E, size=k, replace=False)
    return ids


def zipf_probs(E: int, s: float) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


def draw_routing_zipf(seed: int, T: int, E: int = EXPERTS, k: int = TOPK, s: float = 1.1) -> np.ndarray:
    """k distinct experts per token; rank r has probability proportional to r^-s."""
    g = _rng(seed, _TAG_IDS)
    perm = _rng(seed, _TAG_PERM).permutation(E).astype(np.int32)  # rank -> expert id
    logp = np.log(zipf_probs(E, s))
    ids = np.empty((T, k), dtype=np.int32)
    chunk = 4096
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        gum = g.gumbel(size=(t1 - t0, E))
        keys = logp[None, :] + gum
        top = np.argpartition(-keys, k - 1, axis=1)[:, :k]
        order = np.argsort(-np.take_along_axis(keys, top, axis=1), axis=1, kind="stable")
        ranks = np.take_along_axis(top, order, axis=1)
        ids[t0:t1] = perm[ranks]
    return ids


def draw_router_weights(seed: int, T: int, k: int = TOPK) -> np.ndarray:
    g = _rng(seed, _TAG_W)
    logits = g.standard_normal((T, k)).astype(np.float32)
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m, dtype=np.float32)
    return (ex / ex.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


@dataclass
class Workload:
    name: str
    T: int
    x: np.ndarray          # uint16 bf16 bits [T][H] (fp32 for the single-expert case)
    ids: np.ndarray        # int32 [T][k]
    w: np.ndarray          # float32 [T][k]
    seed: int
    act: str = "bf16"      # "bf16" or "w4a8"
    out_dtype: str = "f32"


# The five configurations: single-expert linear, decode 1 token, decode/verify
# 4 tokens, prefill 8192 tokens (bf16), W4A8 prefill 32768 tokens.
CONFIGS = {
    0: dict(name="linear_4x64x128"),
    1: dict(name="decode_t1_uniform", T=1, routing="uniform", out="f32", act="bf16"),
    2: dict(name="decode_t4_zipf", T=4, routing="zipf", out="f32", act="bf16"),
    3: dict(name="prefill_t8192_zipf", T=8192, routing="zipf", out="bf16", act="bf16", outliers=0.001),
    4: dict(name="prefill_w4a8_t32768_zipf", T=32768, routing="zipf", out="bf16", act="w4a8"),
}


def draw_linear_case(index: int = 0):
    """Single expert: x fp32 N(0,1) [4][128], W [64][128] NVFP4, gamma = fp32(1/2688)."""
    seed = config_seed(index)
    g = _rng(seed, _TAG_X)
    x = g.standard_normal((4, 128)).astype(np.float32)
    codes, scales = draw_proj_expert(seed, "gate", 0, 64, 128)
    gamma = np.array([1.0 / 2688.0], dtype=np.float32)
    return x, codes, scales, gamma


def draw_workload(index: int, T: Optional[int] = None, H: int = HIDDEN, E: int = EXPERTS, k: int = TOPK) -> Workload:
    c = CONFIGS[index]
    seed = config_seed(index)
    T = c["T"] if T is None else T
    x = draw_activations(seed, T, H, c.get("outliers", 0.0))
    if c["routing"] == "uniform":
        ids = draw_routing_uniform(seed, T, E, k)
    else:
        ids = draw_routing_zipf(seed, T, E, k)
    w = draw_router_weights(seed, T, k)
    return Workload(c["name"], T, x, ids, w, seed, c["act"], c["out"])
