"""Thin ctypes binding of libqmoe.so (include/qmoe.h), same call names.

This module only marshals arguments: torch tensors supply device memory and
the current HIP stream; every step of the layer runs in the library's HIP
kernels.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .shapes import SCHEME_CODE

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmoe.so")

QMOE_OK, QMOE_ERR_INVALID_ARG, QMOE_ERR_UNSUPPORTED, QMOE_ERR_HIP = 0, 1, 2, 3
QMOE_DT_BF16, QMOE_DT_F32 = 0, 1
QMOE_FLAG_DUMP_ACC = 1
QMOE_FLAG_PREPACKED = 2
# QMOE_ABI_VERSION of the include/qmoe.h this binding follows; loading a
# library that reports another version fails.
ABI_VERSION = 4

# Every symbol include/qmoe.h declares.
EXPORTS = (
    "qmoe_abi_version", "qmoe_status_str", "qmoe_last_hip_error", "qmoe_route",
    "qmoe_align_capacity", "qmoe_align_workspace", "qmoe_align", "qmoe_check_flags",
    "qmoe_align_noalloc", "qmoe_route_align", "qmoe_default_block_m",
    "qmoe_grouped_ffn_workspace", "qmoe_grouped_ffn_debug_offsets", "qmoe_grouped_ffn",
    "qmoe_grouped_ffn_profiled", "qmoe_combine", "qmoe_prepack", "qmoe_decode_workspace",
    "qmoe_decode",
)
# Largest batch qmoe_decode takes (QMOE_DECODE_MAX_TOKENS).
DECODE_MAX_TOKENS = 16
# Batches up to this size take the one-launch qmoe_decode in moe_forward's
# automatic choice: measured on one MI355X for the 512-expert top-10 a8w4
# block (both paths on the same box), the one launch is faster at 1, 2 and
# 4 tokens (42.3 against 47.1 us, 58.2 against 64.9 us, 85.6 against 87.1
# us), level at 3 (72.1 against 71.6 us), slower from 6 tokens on (114.2
# against 111.2 us; 8 tokens 140.5 against 132.2 us), where the grouped
# kernels stream the weights at a higher rate.
DECODE_PREFERRED_MAX_TOKENS = 4


class QmoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib().qmoe_status_str(status).decode()} (status {status})")


class FfnDesc(ctypes.Structure):
    _fields_ = [("scheme", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class Weights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


_LIB: Optional[ctypes.CDLL] = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
                           "g.build()'` or `python -m quantized_mixture_experts_moe_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.qmoe_abi_version.restype = ctypes.c_int
    if L.qmoe_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} reports ABI version {L.qmoe_abi_version()}, this "
                           f"binding expects {ABI_VERSION}; rebuild the library")
    L.qmoe_status_str.restype = ctypes.c_char_p
    L.qmoe_status_str.argtypes = [ctypes.c_int]
    L.qmoe_last_hip_error.restype = ctypes.c_int
    L.qmoe_route.restype = ctypes.c_int
    L.qmoe_route.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    L.qmoe_align_capacity.restype = sz
    L.qmoe_align_capacity.argtypes = [i32, i32, i32, i32]
    L.qmoe_align_workspace.restype = sz
    L.qmoe_align_workspace.argtypes = [i32, i32, i32]
    L.qmoe_align.restype = ctypes.c_int
    L.qmoe_align.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.qmoe_default_block_m.restype = ctypes.c_int32
    L.qmoe_default_block_m.argtypes = [i32, i32, i32, i32, i32, i32]
    L.qmoe_route_align.restype = ctypes.c_int
    L.qmoe_route_align.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.qmoe_align_noalloc.restype = ctypes.c_int
    L.qmoe_align_noalloc.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.qmoe_check_flags.restype = ctypes.c_int
    L.qmoe_check_flags.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), vp]
    L.qmoe_grouped_ffn_workspace.restype = sz
    L.qmoe_grouped_ffn_workspace.argtypes = [ctypes.POINTER(FfnDesc)]
    L.qmoe_grouped_ffn_debug_offsets.restype = ctypes.c_int
    L.qmoe_grouped_ffn_debug_offsets.argtypes = [ctypes.POINTER(FfnDesc),
                                                 ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.qmoe_grouped_ffn.restype = ctypes.c_int
    L.qmoe_grouped_ffn.argtypes = [ctypes.POINTER(FfnDesc), vp, vp, ctypes.POINTER(Weights),
                                   vp, vp, vp, vp, vp, sz, vp]
    L.qmoe_grouped_ffn_profiled.restype = ctypes.c_int
    L.qmoe_grouped_ffn_profiled.argtypes = [ctypes.POINTER(FfnDesc), vp, vp,
                                            ctypes.POINTER(Weights), vp, vp, vp, vp, vp, sz,
                                            ctypes.POINTER(ctypes.c_void_p), vp]
    L.qmoe_combine.restype = ctypes.c_int
    L.qmoe_combine.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp]
    L.qmoe_prepack.restype = ctypes.c_int
    L.qmoe_prepack.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.qmoe_decode_workspace.restype = sz
    L.qmoe_decode_workspace.argtypes = [ctypes.POINTER(FfnDesc)]
    L.qmoe_decode.restype = ctypes.c_int
    L.qmoe_decode.argtypes = [ctypes.POINTER(FfnDesc), vp, vp, vp, ctypes.POINTER(Weights), vp,
                              vp, vp, vp, vp, vp, sz, vp]
    _LIB = L
    return L


def lib() -> ctypes.CDLL:
    return _lib()


def _check(status: int, what: str):
    if status != QMOE_OK:
        raise QmoeError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libqmoe must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libqmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- routing

def route(logits: torch.Tensor, k: int, ids: Optional[torch.Tensor] = None,
          w: Optional[torch.Tensor] = None):
    """qmoe_route: (topk_ids int32 [T,k], topk_w fp32 [T,k])."""
    T, E = logits.shape
    assert logits.dtype == torch.float32
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(_lib().qmoe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(logits.device)),
           "qmoe_route")
    return ids, w


# ---------------------------------------------------------------- align

def align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return int(_lib().qmoe_align_capacity(T, k, E, block_m))


def align_workspace(T: int, k: int, E: int) -> int:
    return int(_lib().qmoe_align_workspace(T, k, E))


def align(topk_ids: torch.Tensor, E: int, block_m: int, ws: Optional[torch.Tensor] = None,
          out: Optional[dict] = None) -> dict:
    """qmoe_align: expert-sorted, block_m-padded pair slots (``out`` reuses a
    previous result's buffers)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    cap = align_capacity(T, k, E, block_m)
    if out is None:
        out = {
            "sorted_pair_ids": torch.empty(cap, dtype=torch.int32, device=dev),
            "tile_expert": torch.empty(cap // block_m, dtype=torch.int32, device=dev),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "num_padded": torch.empty(1, dtype=torch.int32, device=dev),
            "block_m": block_m,
        }
        ws = out.get("ws", ws)
    else:
        ws = out["ws"]
    need = align_workspace(T, k, E)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    out["ws"] = ws
    _check(_lib().qmoe_align(_ptr(topk_ids), T, k, E, block_m, _ptr(out["sorted_pair_ids"]),
                             _ptr(out["tile_expert"]), _ptr(out["expert_offsets"]),
                             _ptr(out["num_padded"]), _ptr(ws), ws.numel(), _stream(dev)),
           "qmoe_align")
    return out


def route_align(logits: torch.Tensor, k: int, block_m: int, ids=None, w=None,
                out: Optional[dict] = None):
    """qmoe_route_align: (topk_ids, topk_w, grouping dict) in one call (one
    launch up to 16 tokens); ``out`` reuses a previous grouping's buffers."""
    T, E = logits.shape
    assert logits.dtype == torch.float32
    dev = logits.device
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
    cap = align_capacity(T, k, E, block_m)
    if out is None:
        out = {
            "sorted_pair_ids": torch.empty(cap, dtype=torch.int32, device=dev),
            "tile_expert": torch.empty(cap // block_m, dtype=torch.int32, device=dev),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "num_padded": torch.empty(1, dtype=torch.int32, device=dev),
            "block_m": block_m,
        }
    need = align_workspace(T, k, E)
    ws = out.get("ws")
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    out["ws"] = ws
    _check(_lib().qmoe_route_align(_ptr(logits), T, E, k, block_m, _ptr(ids), _ptr(w),
                                   _ptr(out["sorted_pair_ids"]), _ptr(out["tile_expert"]),
                                   _ptr(out["expert_offsets"]), _ptr(out["num_padded"]),
                                   _ptr(ws), ws.numel(), _stream(dev)), "qmoe_route_align")
    return ids, w, out


def align_noalloc(topk_ids: torch.Tensor, E: int, block_m: int, out: Optional[dict] = None,
                  flags: Optional[torch.Tensor] = None) -> dict:
    """qmoe_align_noalloc: the outputs of qmoe_align with the workspace held
    inside the library (``out`` reuses a previous result's buffers; ``flags``
    is an optional int32 device tensor of one element for the flag word)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    cap = align_capacity(T, k, E, block_m)
    if out is None:
        out = {
            "sorted_pair_ids": torch.empty(cap, dtype=torch.int32, device=dev),
            "tile_expert": torch.empty(cap // block_m, dtype=torch.int32, device=dev),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "num_padded": torch.empty(1, dtype=torch.int32, device=dev),
            "block_m": block_m,
        }
    _check(_lib().qmoe_align_noalloc(_ptr(topk_ids), T, k, E, block_m,
                                     _ptr(out["sorted_pair_ids"]), _ptr(out["tile_expert"]),
                                     _ptr(out["expert_offsets"]), _ptr(out["num_padded"]),
                                     _ptr(flags), _stream(dev)), "qmoe_align_noalloc")
    return out


def check_flags(align_ws: torch.Tensor) -> int:
    v = ctypes.c_int32(0)
    _check(_lib().qmoe_check_flags(_ptr(align_ws), ctypes.byref(v), _stream(align_ws.device)),
           "qmoe_check_flags")
    return int(v.value)


# ---------------------------------------------------------------- grouped FFN

def make_desc(scheme: str, T: int, H: int, I: int, E: int, k: int, block_m: int,
              flags: int = 0) -> FfnDesc:
    return FfnDesc(SCHEME_CODE[scheme], T, H, I, E, k, block_m, flags)


def grouped_ffn_workspace(desc: FfnDesc) -> int:
    return int(_lib().qmoe_grouped_ffn_workspace(ctypes.byref(desc)))


def grouped_ffn_debug_offsets(desc: FfnDesc):
    a1, a2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib().qmoe_grouped_ffn_debug_offsets(ctypes.byref(desc), ctypes.byref(a1),
                                                 ctypes.byref(a2)), "debug offsets")
    return int(a1.value), int(a2.value)


def prepack(scheme: str, codes: torch.Tensor, scales: torch.Tensor):
    """qmoe_prepack of one stacked weight tensor (codes [E, N, K bytes]);
    returns (codes, scales) in the streaming layout, same shapes and dtypes.
    W8A8 scales are per-channel and stay as they are (returned as given)."""
    E, N = codes.shape[0], codes.shape[1]
    K = codes.shape[2] * (1 if scheme == "w8a8" else 2)
    c_out = torch.empty_like(codes)
    s_out = scales if scheme == "w8a8" else torch.empty_like(scales)
    _check(_lib().qmoe_prepack(SCHEME_CODE[scheme], E, N, K, _ptr(codes), _ptr(scales),
                               _ptr(c_out), None if scheme == "w8a8" else _ptr(s_out),
                               _stream(codes.device)), "qmoe_prepack")
    return c_out, s_out


def prepack_weights(scheme: str, weights: dict) -> dict:
    """Both projections of a weight dict in the streaming layout; the
    returned dict carries prepacked=True, which grouped_ffn turns into
    QMOE_FLAG_PREPACKED."""
    w13, w13s = prepack(scheme, weights["w13"], weights["w13_scale"])
    w2, w2s = prepack(scheme, weights["w2"], weights["w2_scale"])
    return {"w13": w13, "w13_scale": w13s, "w2": w2, "w2_scale": w2s, "prepacked": True}


def grouped_ffn(scheme: str, x: torch.Tensor, x_scale: Optional[torch.Tensor], weights: dict,
                al: dict, E: int, k: int, flags: int = 0, ws: Optional[torch.Tensor] = None,
                y_pairs: Optional[torch.Tensor] = None, stage_events=None):
    """qmoe_grouped_ffn (qmoe_grouped_ffn_profiled when four recorded
    torch.cuda.Event objects are given); returns (y_pairs [T*k, H], ws)."""
    T, H = x.shape
    I = weights["w13"].shape[1] // 2
    dev = x.device
    if weights.get("prepacked", False):
        flags |= QMOE_FLAG_PREPACKED
    desc = make_desc(scheme, T, H, I, E, k, al["block_m"], flags)
    need = grouped_ffn_workspace(desc)
    if need == 0:
        raise QmoeError(QMOE_ERR_INVALID_ARG, "qmoe_grouped_ffn_workspace")
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    if y_pairs is None:
        ydt = torch.float32 if scheme == "w8a8" else torch.bfloat16
        y_pairs = torch.empty((T * k, H), dtype=ydt, device=dev)
    w = Weights(_ptr(weights["w13"]), _ptr(weights["w13_scale"]), _ptr(weights["w2"]),
                _ptr(weights["w2_scale"]))
    args = (ctypes.byref(desc), _ptr(x), _ptr(x_scale), ctypes.byref(w),
            _ptr(al["sorted_pair_ids"]), _ptr(al["tile_expert"]), _ptr(al["num_padded"]),
            _ptr(y_pairs), _ptr(ws), ws.numel())
    if stage_events is None:
        _check(_lib().qmoe_grouped_ffn(*args, _stream(dev)), "qmoe_grouped_ffn")
    else:
        ev = (ctypes.c_void_p * 4)(*[e.cuda_event for e in stage_events])
        _check(_lib().qmoe_grouped_ffn_profiled(*args, ev, _stream(dev)),
               "qmoe_grouped_ffn_profiled")
    return y_pairs, ws


# ---------------------------------------------------------------- combine

def combine(y_pairs: torch.Tensor, topk_w: torch.Tensor, want_bf16: bool = True,
            want_f32: bool = False, out_bf16=None, out_f32=None):
    """qmoe_combine; returns (out_bf16 or None, out_f32 or None)."""
    T, k = topk_w.shape
    H = y_pairs.shape[1]
    dev = y_pairs.device
    ydt = QMOE_DT_F32 if y_pairs.dtype == torch.float32 else QMOE_DT_BF16
    if want_bf16 and out_bf16 is None:
        out_bf16 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if want_f32 and out_f32 is None:
        out_f32 = torch.empty((T, H), dtype=torch.float32, device=dev)
    _check(_lib().qmoe_combine(_ptr(y_pairs), ydt, _ptr(topk_w), T, k, H, _ptr(out_bf16),
                               _ptr(out_f32), _stream(dev)), "qmoe_combine")
    return out_bf16, out_f32


# ---------------------------------------------------------------- whole layer

def moe_forward(scheme: str, logits: torch.Tensor, x: torch.Tensor,
                x_scale: Optional[torch.Tensor], weights: dict, k: int, block_m: int,
                flags: int = 0, want_f32: bool = False, fused_routing: bool = False,
                path: str = "grouped") -> dict:
    """route -> align -> grouped_ffn -> combine, all on the current stream
    (``fused_routing``: route and align through qmoe_route_align).
    ``path="auto"`` sends batches of up to DECODE_PREFERRED_MAX_TOKENS tokens
    (without debug flags) to the one-launch qmoe_decode instead; its outputs
    are the same bits."""
    if path not in ("grouped", "auto"):
        raise ValueError(f"path must be 'grouped' or 'auto', not {path!r}")
    if path == "auto" and flags == 0 and 0 < x.shape[0] <= DECODE_PREFERRED_MAX_TOKENS:
        return decode_forward(scheme, logits, x, x_scale, weights, k, want_f32=want_f32)
    E = logits.shape[1]
    if fused_routing:
        ids, w, al = route_align(logits, k, block_m)
    else:
        ids, w = route(logits, k)
        al = align(ids, E, block_m)
    y, ws = grouped_ffn(scheme, x, x_scale, weights, al, E, k, flags=flags)
    out_bf16, out_f32 = combine(y, w, want_bf16=True, want_f32=want_f32)
    return {"topk_ids": ids, "topk_w": w, "align": al, "y_pairs": y, "ws": ws,
            "out": out_bf16, "out_f32": out_f32}


# ---------------------------------------------------------------- one-launch decode

def decode_workspace(scheme: str, H: int, I: int, E: int, k: int, flags: int = 0) -> int:
    """qmoe_decode_workspace (bytes; sized for every T up to DECODE_MAX_TOKENS)."""
    return int(_lib().qmoe_decode_workspace(ctypes.byref(make_desc(scheme, 1, H, I, E, k, 16,
                                                                   flags))))


def decode_forward(scheme: str, logits: torch.Tensor, x: torch.Tensor,
                   x_scale: Optional[torch.Tensor], weights: dict, k: int,
                   want_f32: bool = False, ws: Optional[torch.Tensor] = None,
                   y_pairs: Optional[torch.Tensor] = None, want_y: bool = True,
                   out: Optional[dict] = None) -> dict:
    """qmoe_decode: the whole layer in one launch for T <= DECODE_MAX_TOKENS.
    ``ws`` must come from a previous call (or be zero-filled): the library
    keeps arrival counters in it that each call leaves at zero."""
    T, H = x.shape
    E = logits.shape[1]
    I = weights["w13"].shape[1] // 2
    dev = x.device
    flags = QMOE_FLAG_PREPACKED if weights.get("prepacked", False) else 0
    desc = make_desc(scheme, T, H, I, E, k, 16, flags)
    need = int(_lib().qmoe_decode_workspace(ctypes.byref(desc)))
    if need == 0:
        raise QmoeError(QMOE_ERR_INVALID_ARG if T <= DECODE_MAX_TOKENS else QMOE_ERR_UNSUPPORTED,
                        "qmoe_decode_workspace")
    if ws is None or ws.numel() < need:
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    out = {} if out is None else out
    ids = out.get("topk_ids")
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = out.get("topk_w")
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if want_y and y_pairs is None:
        ydt = torch.float32 if scheme == "w8a8" else torch.bfloat16
        y_pairs = torch.empty((T * k, H), dtype=ydt, device=dev)
    ob = out.get("out")
    if ob is None:
        ob = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    of = out.get("out_f32")
    if want_f32 and of is None:
        of = torch.empty((T, H), dtype=torch.float32, device=dev)
    wts = Weights(_ptr(weights["w13"]), _ptr(weights["w13_scale"]), _ptr(weights["w2"]),
                  _ptr(weights["w2_scale"]))
    _check(_lib().qmoe_decode(ctypes.byref(desc), _ptr(logits), _ptr(x), _ptr(x_scale),
                              ctypes.byref(wts), _ptr(ids), _ptr(w), _ptr(y_pairs), _ptr(ob),
                              _ptr(of) if want_f32 else None, _ptr(ws), ws.numel(),
                              _stream(dev)), "qmoe_decode")
    return {"topk_ids": ids, "topk_w": w, "y_pairs": y_pairs, "ws": ws, "out": ob,
            "out_f32": of if want_f32 else None}

