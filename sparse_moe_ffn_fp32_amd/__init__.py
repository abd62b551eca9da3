"""gpt-oss MoE FFN layer on MI355X: Python binding of the HIP C-ABI library.

Each function marshals torch tensors (device memory) and the current HIP
stream into the C entry point of the same name in include/moe.h. Every step of
the layer runs in the library's gfx950 kernels; this module only allocates
outputs and workspace with torch and checks tensor properties.

bf16 tensors may be passed as torch.bfloat16 or as 16-bit integer tensors
holding bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _native

H = 2880
I = 2880

__all__ = ["MoeError", "workspace_size", "pack_weights", "pack_expert_weights", "route", "permute", "expert_ffn", "gate_up",
           "down_accumulate", "combine", "forward", "forward_mx6", "encode_mx6", "gate_up_mx6", "forward_block", "rmsnorm",
           "MX6_ROW_BYTES", "H", "I"]

MX6_ROW_BYTES = 5888   # two-piece MX FP6 record bytes per activation row


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str):
        msg = _native.lib().moe_status_string(status).decode()
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _check(status: int, fn: str):
    if status != _native.MOE_SUCCESS:
        raise MoeError(status, fn)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtypes, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _stream(*ts: Optional[torch.Tensor]):
    """The current stream of the device every given tensor lives on (one
    device per call: the kernels read all their arguments from it)."""
    dev = ts[0].device
    for t in ts[1:]:
        if t is not None and t.device != dev:
            raise ValueError(f"all tensors of a call must be on one device: {t.device} != {dev}")
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def workspace_size(T: int, E: int, k: int) -> int:
    n = _native.lib().moe_workspace_size(T, E, k)
    if n == 0:
        raise ValueError(f"sizes out of range: T={T} E={E} k={k}")
    return n


def _workspace(T: int, E: int, k: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    need = workspace_size(T, E, k)
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    _dev(ws, "workspace", _U8)
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")
    return ws


def _weights(w13_codes, w13_scales, b13, w2_codes, w2_scales, b2):
    E = w13_codes.shape[0]
    _dev(w13_codes, "w13_codes", _U8, (E, 2 * I, H // 2))
    _dev(w13_scales, "w13_scales", _U8, (E, 2 * I, H // 32))
    _dev(b13, "b13", _BF16, (E, 2 * I))
    _dev(w2_codes, "w2_codes", _U8, (E, H, I // 2))
    _dev(w2_scales, "w2_scales", _U8, (E, H, I // 32))
    _dev(b2, "b2", _BF16, (E, H))
    return E


def pack_weights(codes: torch.Tensor, scales: torch.Tensor):
    """Canonical MXFP4 codes [E,N,1440] / scales [E,N,90] -> packed copies (same shapes)."""
    E, N = codes.shape[0], codes.shape[1]
    _dev(codes, "codes", _U8, (E, N, H // 2))
    _dev(scales, "scales", _U8, (E, N, H // 32))
    pc = torch.empty_like(codes)
    ps = torch.empty_like(scales)
    _check(_native.lib().moe_pack_weights(_ptr(codes), _ptr(scales), E, N, _ptr(pc), _ptr(ps),
                                          _stream(codes, scales)), "moe_pack_weights")
    return pc, ps


def pack_expert_weights(w13_codes, w13_scales, w2_codes, w2_scales):
    """Both expert weight tensors -> (w13_codes, w13_scales, w2_codes, w2_scales) packed."""
    return (*pack_weights(w13_codes, w13_scales), *pack_weights(w2_codes, w2_scales))


def route(x: torch.Tensor, Wr: torch.Tensor, br: torch.Tensor, k: int = 4,
          return_logits: bool = False, workspace: Optional[torch.Tensor] = None,
          ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None):
    """-> (topk_ids int32 [T,k], topk_w fp32 [T,k][, logits fp32 [T,E]])"""
    T = x.shape[0]
    E = Wr.shape[0]
    _dev(x, "x", _BF16, (T, H))
    _dev(Wr, "Wr", _F32, (E, H))
    _dev(br, "br", _F32, (E,))
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _dev(ids, "ids", _I32, (T, k))
    _dev(w, "w", _F32, (T, k))
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if return_logits else None
    ws = _workspace(T, E, k, x.device, workspace)
    _check(_native.lib().moe_route(_ptr(x), _ptr(Wr), _ptr(br), T, E, k, _ptr(ids), _ptr(w),
                                   _ptr(logits), _ptr(ws), ws.numel(),
                                   _stream(x, Wr, br, ids, w, ws)), "moe_route")
    return (ids, w, logits) if return_logits else (ids, w)


def permute(topk_ids: torch.Tensor, E: int, workspace: Optional[torch.Tensor] = None):
    """-> (counts int32 [E], offsets int32 [E+1], sorted_rows int32 [T*k])"""
    T, k = topk_ids.shape
    _dev(topk_ids, "topk_ids", _I32)
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    rows = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = _workspace(T, E, k, dev, workspace)
    _check(_native.lib().moe_permute(_ptr(topk_ids), T, E, k, _ptr(counts), _ptr(offsets),
                                     _ptr(rows), _ptr(ws), ws.numel(), _stream(topk_ids, ws)),
           "moe_permute")
    return counts, offsets, rows


def expert_ffn(x, offsets, sorted_rows, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
               k: int = 4, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """-> y fp32 [T*k, 2880], unweighted expert output of every routed slot."""
    T = x.shape[0]
    _dev(x, "x", _BF16, (T, H))
    E = _weights(w13_codes, w13_scales, b13, w2_codes, w2_scales, b2)
    _dev(offsets, "offsets", _I32, (E + 1,))
    _dev(sorted_rows, "sorted_rows", _I32, (T * k,))
    y = torch.empty((T * k, H), dtype=torch.float32, device=x.device)
    ws = _workspace(T, E, k, x.device, workspace)
    _check(_native.lib().moe_expert_ffn(
        _ptr(x), _ptr(offsets), _ptr(sorted_rows), _ptr(w13_codes), _ptr(w13_scales), _ptr(b13),
        _ptr(w2_codes), _ptr(w2_scales), _ptr(b2), T, E, k, _ptr(y), _ptr(ws), ws.numel(),
        _stream(x, offsets, sorted_rows, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, ws)),
        "moe_expert_ffn")
    return y


def gate_up(x, offsets, sorted_rows, w13_codes, w13_scales, b13, k: int = 4,
            h: Optional[torch.Tensor] = None) -> torch.Tensor:
    """-> h bf16 [T*k, 2880] (as int16 bits), SwiGLU of the gate/up projection
    of every routed slot, in expert-sorted order."""
    T = x.shape[0]
    E = w13_codes.shape[0]
    _dev(x, "x", _BF16, (T, H))
    _dev(w13_codes, "w13_codes", _U8, (E, 2 * I, H // 2))
    _dev(w13_scales, "w13_scales", _U8, (E, 2 * I, H // 32))
    _dev(b13, "b13", _BF16, (E, 2 * I))
    _dev(offsets, "offsets", _I32, (E + 1,))
    _dev(sorted_rows, "sorted_rows", _I32, (T * k,))
    if h is None:
        h = torch.empty((T * k, I), dtype=torch.int16, device=x.device)
    else:
        _dev(h, "h", _BF16, (T * k, I))
    _check(_native.lib().moe_gate_up(
        _ptr(x), _ptr(offsets), _ptr(sorted_rows), _ptr(w13_codes), _ptr(w13_scales), _ptr(b13),
        T, E, k, _ptr(h), _stream(x, offsets, sorted_rows, w13_codes, w13_scales, b13, h)),
        "moe_gate_up")
    return h


def gate_up_mx6(x_records, offsets, sorted_rows, w13_codes, w13_scales, b13, k: int = 4,
                h: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gate_up with the activations as encode_mx6 records uint8 [T, 23, 256]."""
    T = x_records.shape[0]
    E = w13_codes.shape[0]
    _dev(x_records, "x_records", _U8, (T, 23, 256))
    _dev(w13_codes, "w13_codes", _U8, (E, 2 * I, H // 2))
    _dev(w13_scales, "w13_scales", _U8, (E, 2 * I, H // 32))
    _dev(b13, "b13", _BF16, (E, 2 * I))
    _dev(offsets, "offsets", _I32, (E + 1,))
    _dev(sorted_rows, "sorted_rows", _I32, (T * k,))
    if h is None:
        h = torch.empty((T * k, I), dtype=torch.int16, device=x_records.device)
    else:
        _dev(h, "h", _BF16, (T * k, I))
    _check(_native.lib().moe_gate_up_mx6(
        _ptr(x_records), _ptr(offsets), _ptr(sorted_rows), _ptr(w13_codes), _ptr(w13_scales),
        _ptr(b13), T, E, k, _ptr(h),
        _stream(x_records, offsets, sorted_rows, w13_codes, w13_scales, b13, h)), "moe_gate_up_mx6")
    return h


def down_accumulate(h, offsets, sorted_rows, topk_w, w2_codes, w2_scales, b2,
                    out: torch.Tensor, k: int = 4) -> torch.Tensor:
    """out[t] += sum_j topk_w[t, j] * (W2[e] h + b2[e]) over the slots of t; returns out."""
    T = out.shape[0]
    E = w2_codes.shape[0]
    _dev(out, "out", _F32, (T, H))
    _dev(h, "h", _BF16, (T * k, I))
    _dev(topk_w, "topk_w", _F32, (T, k))
    _dev(w2_codes, "w2_codes", _U8, (E, H, I // 2))
    _dev(w2_scales, "w2_scales", _U8, (E, H, I // 32))
    _dev(b2, "b2", _BF16, (E, H))
    _dev(offsets, "offsets", _I32, (E + 1,))
    _dev(sorted_rows, "sorted_rows", _I32, (T * k,))
    _check(_native.lib().moe_down_accumulate(
        _ptr(h), _ptr(offsets), _ptr(sorted_rows), _ptr(topk_w), _ptr(w2_codes), _ptr(w2_scales),
        _ptr(b2), T, E, k, _ptr(out),
        _stream(out, h, offsets, sorted_rows, topk_w, w2_codes, w2_scales, b2)), "moe_down_accumulate")
    return out


def combine(y: torch.Tensor, topk_w: torch.Tensor) -> torch.Tensor:
    """-> out fp32 [T, 2880] = sum_j topk_w[t, j] * y[t*k + j]"""
    T, k = topk_w.shape
    _dev(y, "y", _F32, (T * k, H))
    _dev(topk_w, "topk_w", _F32)
    out = torch.empty((T, H), dtype=torch.float32, device=y.device)
    _check(_native.lib().moe_combine(_ptr(y), _ptr(topk_w), T, k, _ptr(out), _stream(y, topk_w)),
           "moe_combine")
    return out


def forward(x, Wr, br, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, k: int = 4,
            out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer -> out fp32 [T, 2880]."""
    return _forward("moe_forward", x, Wr, br, w13_codes, w13_scales, b13, w2_codes, w2_scales,
                    b2, k, out, workspace)


def forward_mx6(x, Wr, br, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, k: int = 4,
                out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer with the tiled expert GEMMs on the block-scaled FP4 x FP6
    matrix cores (activations as two MX FP6 pieces) -> out fp32 [T, 2880]."""
    return _forward("moe_forward_mx6", x, Wr, br, w13_codes, w13_scales, b13, w2_codes,
                    w2_scales, b2, k, out, workspace)


def encode_mx6(x: torch.Tensor) -> torch.Tensor:
    """bf16 rows [R, 2880] -> two-piece MX FP6 records uint8 [R, 23, 256]."""
    R = x.shape[0]
    _dev(x, "x", _BF16, (R, H))
    rec = torch.empty((R, 23, 256), dtype=torch.uint8, device=x.device)
    _check(_native.lib().moe_encode_mx6(_ptr(x), R, _ptr(rec), _stream(x)), "moe_encode_mx6")
    return rec


def rmsnorm(x: torch.Tensor, scale: torch.Tensor, eps: float = 1e-5) -> torch.Tensor:
    """bf16 rows [T, 2880] -> bf16(x / sqrt(mean(x^2) + eps) * scale), as int16 bits."""
    T = x.shape[0]
    _dev(x, "x", _BF16, (T, H))
    _dev(scale, "scale", _F32, (H,))
    t = torch.empty((T, H), dtype=torch.int16, device=x.device)
    _check(_native.lib().moe_rmsnorm(_ptr(x), _ptr(scale), float(eps), T, _ptr(t),
                                     _stream(x, scale)),
           "moe_rmsnorm")
    return t


def forward_block(x, norm_scale, Wr, br, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                  k: int = 4, norm_eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out fp32 [T, 2880] = x + layer(bf16(RMSNorm(x))): the MoE sublayer of a
    decoder layer with its pre-norm and residual add."""
    T = x.shape[0]
    E = Wr.shape[0]
    _dev(x, "x", _BF16, (T, H))
    _dev(norm_scale, "norm_scale", _F32, (H,))
    _dev(Wr, "Wr", _F32, (E, H))
    _dev(br, "br", _F32, (E,))
    if _weights(w13_codes, w13_scales, b13, w2_codes, w2_scales, b2) != E:
        raise ValueError("router and expert weights disagree on the expert count")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    else:
        _dev(out, "out", _F32, (T, H))
    ws = _workspace(T, E, k, x.device, workspace)
    _check(_native.lib().moe_forward_block(
        _ptr(x), _ptr(norm_scale), float(norm_eps), _ptr(Wr), _ptr(br), _ptr(w13_codes),
        _ptr(w13_scales), _ptr(b13), _ptr(w2_codes), _ptr(w2_scales), _ptr(b2), T, E, k,
        _ptr(out), _ptr(ws), ws.numel(),
        _stream(x, norm_scale, Wr, br, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, out, ws)),
        "moe_forward_block")
    return out


def _forward(fn, x, Wr, br, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, k, out,
             workspace) -> torch.Tensor:
    T = x.shape[0]
    E = Wr.shape[0]
    _dev(x, "x", _BF16, (T, H))
    _dev(Wr, "Wr", _F32, (E, H))
    _dev(br, "br", _F32, (E,))
    if _weights(w13_codes, w13_scales, b13, w2_codes, w2_scales, b2) != E:
        raise ValueError("router and expert weights disagree on the expert count")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    else:
        _dev(out, "out", _F32, (T, H))
    ws = _workspace(T, E, k, x.device, workspace)
    _check(getattr(_native.lib(), fn)(
        _ptr(x), _ptr(Wr), _ptr(br), _ptr(w13_codes), _ptr(w13_scales), _ptr(b13),
        _ptr(w2_codes), _ptr(w2_scales), _ptr(b2), T, E, k, _ptr(out), _ptr(ws), ws.numel(),
        _stream(x, Wr, br, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, out, ws)), fn)
    return out
