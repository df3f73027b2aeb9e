"""ctypes binding of libnvfp4moe.so: the same entry points as include/nvfp4moe.h.

Argument marshalling only: tensors become device pointers, dtypes become the C enums,
and the current torch stream is passed through. No arithmetic of the method is done
here; a non-zero status raises NVFP4Error.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libnvfp4moe.so"

DTYPE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
ACT = {"bf16": 0, "w4a8": 1, "w4a8_f16": 2, "w4a4": 3}
ISA = {"auto": 0, "portable": 1, "avx2": 2, "avx512": 3}

_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class _Weight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("global_", ctypes.c_void_p),
        ("N", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("format", ctypes.c_int32),
    ]


FORMAT = {"nvfp4": 0, "q8_0": 1}


def lib_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


_SIGS = {
    "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4_dequant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "nvfp4_linear": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_Weight),
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "nvfp4_route_workspace_size": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "nvfp4_moe_route": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]),
    "nvfp4_quant_rows_i8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "nvfp4_quant_rows_nvfp4": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "nvfp4_router_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 2),
    "nvfp4_router_topk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "nvfp4_moe_decode_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 5),
    "nvfp4_moe_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(_Weight), ctypes.POINTER(_Weight), ctypes.POINTER(_Weight),
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
    "nvfp4_moe_decode_stage": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.POINTER(_Weight), ctypes.POINTER(_Weight),
                                              ctypes.POINTER(_Weight), ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "nvfp4_moe_prefill_stage": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.POINTER(_Weight), ctypes.POINTER(_Weight),
                                               ctypes.POINTER(_Weight), ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "nvfp4_moe_prefill_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 6),
    "nvfp4_moe_prefill_workspace_region": (ctypes.c_int, [ctypes.c_int32] * 7 + [ctypes.POINTER(ctypes.c_size_t)] * 2),
    "nvfp4_moe_decode_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.POINTER(_Weight), ctypes.POINTER(_Weight),
                                                ctypes.POINTER(_Weight), ctypes.c_int32, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                                ctypes.c_void_p]),
    "nvfp4_host_isa": (ctypes.c_int32, []),
    "nvfp4_moe_decode_host": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(_Weight), ctypes.POINTER(_Weight),
                                             ctypes.POINTER(_Weight), ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]),
    "nvfp4_moe_prefill": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(_Weight), ctypes.POINTER(_Weight), ctypes.POINTER(_Weight),
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "nvfp4_moe_prefill_shared_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 6),
    "nvfp4_moe_prefill_shared": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                                 + [ctypes.POINTER(_Weight)] * 3 + [ctypes.c_int32] + [ctypes.POINTER(_Weight)] * 3
                                 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p]),
    "nvfp4_moe_decode_shared_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 5),
    "nvfp4_moe_decode_shared": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                                + [ctypes.POINTER(_Weight)] * 3 + [ctypes.c_int32] + [ctypes.POINTER(_Weight)] * 3
                                + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
}


def load_library() -> ctypes.CDLL:
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = load_library().nvfp4_status_string(status).decode()
        raise NVFP4Error(fn, status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


@dataclass
class Proj:
    """One NVFP4 projection of E experts on the device: codes uint8 [E][N][K/2],
    scales uint8 [E][N][K/16], gamma float32 [E]."""
    codes: torch.Tensor
    scales: torch.Tensor
    gamma: torch.Tensor

    @property
    def N(self) -> int:
        return int(self.codes.shape[1])

    @property
    def K(self) -> int:
        return int(self.codes.shape[2]) * 2

    fmt = "nvfp4"

    def cstruct(self) -> _Weight:
        return _Weight(_ptr(self.codes), _ptr(self.scales), _ptr(self.gamma), self.N, self.K, FORMAT[self.fmt])

    @staticmethod
    def from_numpy(p, device) -> "Proj":
        if getattr(p, "fmt", "nvfp4") == "q8_0":
            return Q8Proj.from_numpy(p, device)
        return Proj(torch.from_numpy(p.codes).to(device), torch.from_numpy(p.scales).to(device),
                    torch.from_numpy(p.gamma).to(device))


@dataclass
class Q8Proj:
    """One Q8_0 projection of E experts on the device (down projections): codes int8
    [E][N][K], scales fp16 bits (int16) [E][N][K/32], gamma float32 [E] or None (= 1)."""
    codes: torch.Tensor
    scales: torch.Tensor
    gamma: Optional[torch.Tensor] = None
    fmt = "q8_0"

    @property
    def N(self) -> int:
        return int(self.codes.shape[1])

    @property
    def K(self) -> int:
        return int(self.codes.shape[2])

    def cstruct(self) -> _Weight:
        return _Weight(_ptr(self.codes), _ptr(self.scales), _ptr(self.gamma), self.N, self.K, FORMAT[self.fmt])

    @staticmethod
    def from_numpy(p, device, with_gamma: bool = False) -> "Q8Proj":
        return Q8Proj(torch.from_numpy(p.codes).to(device), torch.from_numpy(p.scales.view("int16")).to(device),
                      torch.from_numpy(p.gamma).to(device) if with_gamma else None)


@dataclass
class Layer:
    gate: Proj
    up: Proj
    down: "Proj | Q8Proj"

    @property
    def E(self) -> int:
        return int(self.gate.codes.shape[0])

    @property
    def H(self) -> int:
        return self.gate.K

    @property
    def I(self) -> int:
        return self.gate.N

    @staticmethod
    def from_numpy(layer, device="cuda") -> "Layer":
        return Layer(Proj.from_numpy(layer.gate, device), Proj.from_numpy(layer.up, device),
                     Proj.from_numpy(layer.down, device))


def dequant(codes: torch.Tensor, scales: torch.Tensor, gamma: Optional[torch.Tensor] = None,
            out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """codes [rows][K/2], scales [rows][K/16], gamma: one float32 or None."""
    lib = load_library()
    K = int(codes.shape[-1]) * 2
    rows = codes.numel() // (K // 2)
    if out is None:
        out = torch.empty(codes.shape[:-1] + (K,), dtype=out_dtype, device=codes.device)
    _check("nvfp4_dequant", lib.nvfp4_dequant(_ptr(codes), _ptr(scales), _ptr(gamma), rows, K, DTYPE[out.dtype],
                                              _ptr(out), _stream(codes.device)))
    return out


def linear(x: torch.Tensor, proj: Proj, expert: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load_library()
    T = int(x.shape[0])
    if out is None:
        out = torch.empty((T, proj.N), dtype=torch.float32, device=x.device)
    w = proj.cstruct()
    _check("nvfp4_linear", lib.nvfp4_linear(_ptr(x), DTYPE[x.dtype], T, ctypes.byref(w), expert, _ptr(out),
                                            _stream(x.device)))
    return out


def route_workspace_size(T: int, topk: int, E: int) -> int:
    return int(load_library().nvfp4_route_workspace_size(T, topk, E))


def route(ids: torch.Tensor, E: int, ws: Optional[torch.Tensor] = None):
    """Returns (expert_offsets int32 [E+1], sorted_pairs int32 [T*topk], ws)."""
    lib = load_library()
    T, k = int(ids.shape[0]), int(ids.shape[1])
    dev = ids.device
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    need = route_workspace_size(T, k, E)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("nvfp4_moe_route", lib.nvfp4_moe_route(_ptr(ids), T, k, E, _ptr(off), _ptr(sp), _ptr(ws), ws.numel(),
                                                  _stream(dev)))
    return off, sp[:T * k], ws


def quant_rows_i8(x: torch.Tensor):
    lib = load_library()
    rows, cols = int(x.shape[0]), int(x.shape[1])
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check("nvfp4_quant_rows_i8", lib.nvfp4_quant_rows_i8(_ptr(x), DTYPE[x.dtype], rows, cols, _ptr(q), _ptr(s),
                                                          _stream(x.device)))
    return q, s


def quant_rows_nvfp4(x: torch.Tensor):
    """x [rows][cols] float32 or bfloat16 -> (codes uint8 [rows][cols/2], scales uint8
    [rows][cols/16] E4M3, g float32 [rows]) by the library's per-row NVFP4 rule."""
    lib = load_library()
    rows, cols = int(x.shape[0]), int(x.shape[1])
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check("nvfp4_quant_rows_nvfp4", lib.nvfp4_quant_rows_nvfp4(_ptr(x), DTYPE[x.dtype], rows, cols, _ptr(codes),
                                                                _ptr(scales), _ptr(g), _stream(x.device)))
    return codes, scales, g


def router_workspace_size(T: int, E: int) -> int:
    return int(load_library().nvfp4_router_workspace_size(T, E))


def router_topk(x: torch.Tensor, w_router: torch.Tensor, topk: int, ws: Optional[torch.Tensor] = None):
    """x [T][H] float32 or bfloat16, w_router bf16 [E][H] (bfloat16 or int16 bits).
    Returns (topk_ids int32 [T][topk], topk_weights float32 [T][topk])."""
    lib = load_library()
    T, H = int(x.shape[0]), int(x.shape[1])
    E = int(w_router.shape[0])
    ids = torch.empty((T, topk), dtype=torch.int32, device=x.device)
    wts = torch.empty((T, topk), dtype=torch.float32, device=x.device)
    ws = _ws(ws, router_workspace_size(T, E), x.device)  # zero-filled when new (completion counter)
    _check("nvfp4_router_topk", lib.nvfp4_router_topk(_ptr(x), DTYPE[x.dtype], T, H, _ptr(w_router), E, topk,
                                                      _ptr(ids), _ptr(wts), _ptr(ws), ws.numel(),
                                                      _stream(x.device)))
    return ids, wts


def decode_workspace_size(T: int, H: int, I: int, E: int, topk: int, shared: bool = False) -> int:
    lib = load_library()
    fn = lib.nvfp4_moe_decode_shared_workspace_size if shared else lib.nvfp4_moe_decode_workspace_size
    return int(fn(T, H, I, E, topk))


def prefill_workspace_size(T: int, H: int, I: int, E: int, topk: int, act: str = "bf16",
                           shared: bool = False) -> int:
    lib = load_library()
    fn = lib.nvfp4_moe_prefill_shared_workspace_size if shared else lib.nvfp4_moe_prefill_workspace_size
    return int(fn(T, H, I, E, topk, ACT[act]))


WS_REGION = {"expert_offsets": 0, "sorted_pairs": 1, "pair_position": 2, "x_staged": 3, "x_rowscale": 4,
             "h": 5, "h_exp": 6, "h_q": 7, "h_scale": 8, "y": 9, "x_blockscale": 10, "h_blockscale": 11}


def prefill_workspace_region(T: int, H: int, I: int, E: int, topk: int, act: str, region: str):
    """(byte offset, bytes) of an intermediate result inside a prefill workspace."""
    off, nb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("nvfp4_moe_prefill_workspace_region", load_library().nvfp4_moe_prefill_workspace_region(
        T, H, I, E, topk, ACT[act], WS_REGION[region], ctypes.byref(off), ctypes.byref(nb)))
    return int(off.value), int(nb.value)


DECODE_ERROR_WORD = slice(4, 8)       # bytes of the decode workspace's error flags
DECODE_SPIN_WORD = slice(8, 12)       # bytes of its grid-barrier spin-limit override


def check_decode_workspace(ws: torch.Tensor) -> None:
    """Raise NVFP4Error if a decode call on this workspace reported a grid-barrier timeout
    (its output is then invalid); clears the flag. Synchronizes with the device."""
    word = ws[DECODE_ERROR_WORD].view(torch.int32)
    flags = int(word.item())
    if flags & 1:
        word.zero_()
        raise NVFP4Error("nvfp4_moe_decode", flags, "grid barrier timed out: the output is invalid")


def _ws(ws: Optional[torch.Tensor], need: int, dev) -> torch.Tensor:
    """A workspace of at least `need` bytes; new ones are zero-filled (the decode
    workspace holds a grid-barrier counter that must start at zero)."""
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    return ws


def moe_decode(x: torch.Tensor, layer: Layer, ids: torch.Tensor, w: torch.Tensor,
               out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, check: bool = True,
               shared: Optional[Layer] = None) -> torch.Tensor:
    """check: read the workspace's error word after the call (a device synchronization)
    and raise if the grid barrier timed out; launch loops pass False and call
    check_decode_workspace() when they use a result. shared: the layer's shared expert (a
    one-expert Layer), applied to every token with weight 1 (nvfp4_moe_decode_shared)."""
    lib = load_library()
    T, H = int(x.shape[0]), int(x.shape[1])
    k = int(ids.shape[1])
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    ws = _ws(ws, decode_workspace_size(T, H, layer.I, layer.E, k, shared=shared is not None), x.device)
    g, u, d = layer.gate.cstruct(), layer.up.cstruct(), layer.down.cstruct()
    if shared is None:
        _check("nvfp4_moe_decode", lib.nvfp4_moe_decode(
            _ptr(x), DTYPE[x.dtype], T, H, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), layer.E, _ptr(ids),
            _ptr(w), k, _ptr(out), DTYPE[out.dtype], _ptr(ws), ws.numel(), _stream(x.device)))
    else:
        sg, su, sd = shared.gate.cstruct(), shared.up.cstruct(), shared.down.cstruct()
        _check("nvfp4_moe_decode_shared", lib.nvfp4_moe_decode_shared(
            _ptr(x), DTYPE[x.dtype], T, H, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), layer.E,
            ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), _ptr(ids), _ptr(w), k, _ptr(out),
            DTYPE[out.dtype], _ptr(ws), ws.numel(), _stream(x.device)))
    if check and T > 0:
        check_decode_workspace(ws)
    return out


def _host_args(x, ids, w, out):
    """The host entry point reads x, ids and w and writes T*H floats to out as host memory:
    check devices, dtypes and shapes before handing it the pointers."""
    T = int(x.shape[0])
    for name, t in (("x", x), ("ids", ids), ("w", w), ("out", out)):
        if t is not None and t.device.type != "cpu":
            raise ValueError(f"{name} must be a CPU tensor for the host decode path (got {t.device})")
    if x.dim() != 2 or x.dtype not in DTYPE:
        raise ValueError("x must be a [T][H] tensor of a library dtype")
    if ids.dim() != 2 or ids.dtype != torch.int32 or int(ids.shape[0]) != T:
        raise ValueError("ids must be an int32 [T][topk] tensor")
    if w.dtype != torch.float32 or tuple(w.shape) != tuple(ids.shape):
        raise ValueError("w must be a float32 [T][topk] tensor")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (T, int(x.shape[1]))):
        raise ValueError("out must be a float32 [T][H] tensor")


def moe_decode_noalloc(x: torch.Tensor, layer: Layer, ids: torch.Tensor, w: torch.Tensor,
                       out: torch.Tensor) -> torch.Tensor:
    """nvfp4_moe_decode_noalloc: the decode with the library's static device scratch as its
    workspace (no workspace argument; out must be given)."""
    lib = load_library()
    T, H = int(x.shape[0]), int(x.shape[1])
    g, u, d = layer.gate.cstruct(), layer.up.cstruct(), layer.down.cstruct()
    _check("nvfp4_moe_decode_noalloc", lib.nvfp4_moe_decode_noalloc(
        _ptr(x), DTYPE[x.dtype], T, H, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), layer.E, _ptr(ids),
        _ptr(w), int(ids.shape[1]), _ptr(out), DTYPE[out.dtype], _stream(x.device)))
    return out


def host_isa() -> str:
    """The widest instruction set the host row kernels can use on this CPU."""
    code = int(load_library().nvfp4_host_isa())
    return next(k for k, v in ISA.items() if v == code)


def moe_decode_host(x: torch.Tensor, layer: Layer, ids: torch.Tensor, w: torch.Tensor, n_threads: int = 0,
                    isa: str = "auto", out: Optional[torch.Tensor] = None):
    """The routed-expert projection on the host CPU: every tensor (the layer's too) in host
    memory; x [T][H] float32 or bfloat16; returns (out float32 [T][H], dropped pairs)."""
    lib = load_library()
    _host_args(x, ids, w, out)
    T, H = int(x.shape[0]), int(x.shape[1])
    k = int(ids.shape[1])
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32)
    g, u, d = layer.gate.cstruct(), layer.up.cstruct(), layer.down.cstruct()
    dropped = ctypes.c_int64(0)
    _check("nvfp4_moe_decode_host", lib.nvfp4_moe_decode_host(
        _ptr(x), DTYPE[x.dtype], T, H, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), layer.E, _ptr(ids),
        _ptr(w), k, _ptr(out), n_threads, ISA[isa], ctypes.byref(dropped)))
    return out, int(dropped.value)


def moe_prefill(x: torch.Tensor, layer: Layer, ids: torch.Tensor, w: torch.Tensor, act: str = "bf16",
                out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, shared: Optional[Layer] = None) -> torch.Tensor:
    """shared: the layer's shared expert (a one-expert Layer), applied to every token with
    weight 1 in the same launches (nvfp4_moe_prefill_shared)."""
    lib = load_library()
    T, H = int(x.shape[0]), int(x.shape[1])
    k = int(ids.shape[1])
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    ws = _ws(ws, prefill_workspace_size(T, H, layer.I, layer.E, k, act, shared=shared is not None), x.device)
    g, u, d = layer.gate.cstruct(), layer.up.cstruct(), layer.down.cstruct()
    if shared is None:
        _check("nvfp4_moe_prefill", lib.nvfp4_moe_prefill(
            _ptr(x), DTYPE[x.dtype], T, H, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), layer.E, _ptr(ids),
            _ptr(w), k, ACT[act], _ptr(out), DTYPE[out.dtype], _ptr(ws), ws.numel(), _stream(x.device)))
    else:
        sg, su, sd = shared.gate.cstruct(), shared.up.cstruct(), shared.down.cstruct()
        _check("nvfp4_moe_prefill_shared", lib.nvfp4_moe_prefill_shared(
            _ptr(x), DTYPE[x.dtype], T, H, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), layer.E,
            ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), _ptr(ids), _ptr(w), k, ACT[act], _ptr(out),
            DTYPE[out.dtype], _ptr(ws), ws.numel(), _stream(x.device)))
    return out


class PreparedCall:
    """A decode or prefill call with its arguments marshalled once, for launch loops
    (benchmarks, graph capture): run() enqueues the whole call, stage(i) one stage."""

    def __init__(self, kind: str, x, layer: Layer, ids, w, out, ws, act: str = "bf16",
                 shared: Optional[Layer] = None):
        self.lib = load_library()
        self.kind = kind
        self.keep = (x, layer, ids, w, out, ws, shared)
        self._w = (layer.gate.cstruct(), layer.up.cstruct(), layer.down.cstruct())
        g, u, d = (ctypes.byref(v) for v in self._w)
        T, H = int(x.shape[0]), int(x.shape[1])
        k = int(ids.shape[1])
        tail = [_ptr(out), DTYPE[out.dtype], _ptr(ws), ws.numel()]
        self.device = x.device
        if shared is not None:
            # the shared-expert entry points have no staged form
            self._s = (shared.gate.cstruct(), shared.up.cstruct(), shared.down.cstruct())
            sg, su, sd = (ctypes.byref(v) for v in self._s)
            common = [_ptr(x), DTYPE[x.dtype], T, H, g, u, d, layer.E, sg, su, sd, _ptr(ids), _ptr(w), k]
            self.staged, self.nstages = None, 0
            if kind == "decode":
                self.args, self.full = common + tail, self.lib.nvfp4_moe_decode_shared
            else:
                self.args, self.full = common + [ACT[act]] + tail, self.lib.nvfp4_moe_prefill_shared
            return
        common = [_ptr(x), DTYPE[x.dtype], T, H, g, u, d, layer.E, _ptr(ids), _ptr(w), k]
        if kind == "decode":
            self.args = common + tail
            self.full, self.staged, self.nstages = self.lib.nvfp4_moe_decode, self.lib.nvfp4_moe_decode_stage, 2
        else:
            self.args = common + [ACT[act]] + tail
            self.full, self.staged, self.nstages = self.lib.nvfp4_moe_prefill, self.lib.nvfp4_moe_prefill_stage, 4

    def run(self) -> None:
        # the stream is looked up per call, so graph capture sees its capture stream
        _check(self.kind, self.full(*self.args, _stream(self.device)))

    def stage(self, i: int) -> None:
        if self.staged is None:
            raise NVFP4Error(self.kind + "_stage", -1, "the shared-expert calls have no staged form")
        _check(self.kind + "_stage", self.staged(i, *self.args, _stream(self.device)))

    def check(self) -> None:
        """Decode: raise if a call since the last check reported a grid-barrier timeout."""
        if self.kind == "decode":
            check_decode_workspace(self.keep[5])


class PreparedHostCall:
    """A host-CPU decode call (nvfp4_moe_decode_host) with its arguments marshalled once,
    for call loops: run() runs the call on the CPU threads and returns the dropped count."""

    def __init__(self, x, layer: Layer, ids, w, out, n_threads: int = 0, isa: str = "auto"):
        self.lib = load_library()
        _host_args(x, ids, w, out)
        if out is None:
            raise ValueError("out must be given")
        self.keep = (x, layer, ids, w, out)
        self._w = (layer.gate.cstruct(), layer.up.cstruct(), layer.down.cstruct())
        self._dropped = ctypes.c_int64(0)
        g, u, d = (ctypes.byref(v) for v in self._w)
        T, H = int(x.shape[0]), int(x.shape[1])
        self.args = [_ptr(x), DTYPE[x.dtype], T, H, g, u, d, layer.E, _ptr(ids), _ptr(w), int(ids.shape[1]),
                     _ptr(out), n_threads, ISA[isa], ctypes.byref(self._dropped)]

    def run(self) -> int:
        _check("nvfp4_moe_decode_host", self.lib.nvfp4_moe_decode_host(*self.args))
        return int(self._dropped.value)
