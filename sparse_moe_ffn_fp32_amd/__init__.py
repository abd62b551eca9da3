"""gpt-oss MoE FFN layer on MI355X: Python binding of the HIP C-ABI library.

Each function marshals torch tensors (device memory) and the current HIP
stream into the C entry point of the same name in include/moe.h. Every step of
the layer runs in the library's gfx950 kernels; this module only allocates
outputs and workspace with torch and checks tensor properties.

The expert weights enter the layer calls only as a PackedExperts (from
pack_experts), whose packed MXFP4 tensors have shapes of their own
([E, N/64, 92160] codes, [E, N/64, 5760] scales) and carry the descriptor the
library's pack call filled; checkpoint-layout code and scale tensors are
refused.

bf16 tensors may be passed as torch.bfloat16 or as 16-bit integer tensors
holding bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Optional

import torch

from . import _native

H = 2880
I = 2880

__all__ = ["MoeError", "PackedWeight", "PackedExperts", "workspace_size", "workspace_routing", "pack_weights",
           "pack_experts", "route", "permute", "expert_ffn", "gate_up", "down_accumulate",
           "combine", "forward", "forward_mx6", "encode_mx6", "gate_up_mx6", "forward_block",
           "rmsnorm", "forward_noalloc", "MX6_ROW_BYTES", "H", "I"]

MX6_ROW_BYTES = 5888   # two-piece MX FP6 record bytes per activation row
_GROUP_CODE_BYTES = 64 * (H // 2)    # packed codes of one 64-row group
_GROUP_SCALE_BYTES = 64 * (H // 32)  # packed scales of one 64-row group


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


@dataclass(eq=False)
class PackedWeight:
    """One MXFP4 weight tensor [E, N, 2880] in the library's packed order:
    codes uint8 [E, N/64, 92160], scales uint8 [E, N/64, 5760], and the
    moe_packed_weight_t descriptor the pack call filled. Made by pack_weights."""
    codes: torch.Tensor
    scales: torch.Tensor
    E: int
    N: int
    _desc: _native.PackedWeightDesc = field(repr=False)

    def desc(self):
        """The C descriptor, checked to still describe these tensors."""
        d = self._desc
        if (d.tag != _native.MOE_PACKED_TAG or d.codes != self.codes.data_ptr()
                or d.scales != self.scales.data_ptr() or d.E != self.E or d.N != self.N):
            raise ValueError("packed weight descriptor no longer matches its tensors")
        return ctypes.byref(d)

    @property
    def scale_spread(self) -> int:
        """Largest spread (max - min, in binades) of the E8M0 scale exponents
        within one expert; the FP6-piece path refuses more than
        MOE_MX6_MAX_SCALE_SPREAD."""
        return int(self._desc.scale_spread)


@dataclass(eq=False)
class PackedExperts:
    """The expert weights of one layer as the expert GEMMs take them:
    w13 (gate/up, N = 5760, rows interleaved gate/up) and w2 (down, N = 2880)
    packed, and their bf16 biases b13 [E, 5760], b2 [E, 2880]."""
    w13: PackedWeight
    b13: torch.Tensor
    w2: PackedWeight
    b2: torch.Tensor

    @property
    def E(self) -> int:
        return self.w13.E

    def tensors(self):
        return (self.w13.codes, self.w13.scales, self.b13, self.w2.codes, self.w2.scales, self.b2)


def _experts(experts, E: Optional[int] = None) -> PackedExperts:
    if not isinstance(experts, PackedExperts):
        raise TypeError("expert weights must be a PackedExperts (from pack_experts); "
                        "raw code / scale tensors are not accepted")
    if experts.w13.N != 2 * I or experts.w2.N != H or experts.w2.E != experts.w13.E:
        raise ValueError("PackedExperts: w13 must have 5760 rows, w2 2880, and the same experts")
    _dev(experts.b13, "b13", _BF16, (experts.E, 2 * I))
    _dev(experts.b2, "b2", _BF16, (experts.E, H))
    if E is not None and experts.E != E:
        raise ValueError(f"router has {E} experts, the expert weights {experts.E}")
    return experts


def workspace_size(T: int, E: int, k: int, op: Optional[str] = None) -> int:
    """Workspace bytes of entry point `op` ('route', 'permute', 'expert_ffn',
    'forward', 'forward_mx6', 'forward_block'); None: enough for any."""
    if op is None:
        n = _native.lib().moe_workspace_size(T, E, k)
    else:
        n = _native.lib().moe_workspace_size_op(_native.OPS[op], T, E, k)
    if n == 0:
        raise ValueError(f"sizes out of range: T={T} E={E} k={k}")
    return n


def workspace_routing(workspace: torch.Tensor, T: int, k: int):
    """The routing a layer call leaves at the head of its workspace
    (include/moe.h): expert ids int32 [T, k] and weights fp32 [T, k], as views."""
    _dev(workspace, "workspace", _U8)
    n = T * k
    w_off = (n * 4 + 255) // 256 * 256
    if workspace.numel() < w_off + n * 4:
        raise ValueError("workspace too small for the routing of T tokens")
    ids = workspace[: n * 4].view(torch.int32).view(T, k)
    w = workspace[w_off: w_off + n * 4].view(torch.float32).view(T, k)
    return ids, w


def _workspace(T: int, E: int, k: int, device, ws: Optional[torch.Tensor], op: str) -> torch.Tensor:
    need = workspace_size(T, E, k, op)
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    _dev(ws, "workspace", _U8)
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")
    return ws


def pack_weights(codes: torch.Tensor, scales: torch.Tensor) -> PackedWeight:
    """Canonical MXFP4 codes [E,N,1440] / scales [E,N,90] -> PackedWeight."""
    E, N = codes.shape[0], codes.shape[1]
    _dev(codes, "codes", _U8, (E, N, H // 2))
    _dev(scales, "scales", _U8, (E, N, H // 32))
    if N % 64:
        raise ValueError(f"rows per expert must be a multiple of 64, got {N}")
    pc = torch.empty((E, N // 64, _GROUP_CODE_BYTES), dtype=torch.uint8, device=codes.device)
    ps = torch.empty((E, N // 64, _GROUP_SCALE_BYTES), dtype=torch.uint8, device=codes.device)
    d = _native.PackedWeightDesc()
    _check(_native.lib().moe_pack_weights(_ptr(codes), _ptr(scales), E, N, _ptr(pc), _ptr(ps),
                                          ctypes.byref(d), _stream(codes, scales)),
           "moe_pack_weights")
    return PackedWeight(pc, ps, E, N, d)


def pack_experts(w13_codes, w13_scales, b13, w2_codes, w2_scales, b2) -> PackedExperts:
    """Checkpoint-layout expert weights -> PackedExperts (one-time packing)."""
    E = w13_codes.shape[0]
    _dev(b13, "b13", _BF16, (E, 2 * I))
    _dev(b2, "b2", _BF16, (E, H))
    w13 = pack_weights(w13_codes, w13_scales)
    w2 = pack_weights(w2_codes, w2_scales)
    if w13.N != 2 * I or w2.N != H or w2.E != E:
        raise ValueError("w13 must be [E, 5760, ...] and w2 [E, 2880, ...]")
    return PackedExperts(w13, b13, w2, b2)


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
    ws = _workspace(T, E, k, x.device, workspace, "route")
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
    ws = _workspace(T, E, k, dev, workspace, "permute")
    _check(_native.lib().moe_permute(_ptr(topk_ids), T, E, k, _ptr(counts), _ptr(offsets),
                                     _ptr(rows), _ptr(ws), ws.numel(), _stream(topk_ids, ws)),
           "moe_permute")
    return counts, offsets, rows


def expert_ffn(x, offsets, sorted_rows, experts: PackedExperts, k: int = 4,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """-> y fp32 [T*k, 2880], unweighted expert output of every routed slot."""
    T = x.shape[0]
    _dev(x, "x", _BF16, (T, H))
    ex = _experts(experts)
    E = ex.E
    _dev(offsets, "offsets", _I32, (E + 1,))
    _dev(sorted_rows, "sorted_rows", _I32, (T * k,))
    y = torch.empty((T * k, H), dtype=torch.float32, device=x.device)
    ws = _workspace(T, E, k, x.device, workspace, "expert_ffn")
    _check(_native.lib().moe_expert_ffn(
        _ptr(x), _ptr(offsets), _ptr(sorted_rows), ex.w13.desc(), _ptr(ex.b13), ex.w2.desc(),
        _ptr(ex.b2), T, E, k, _ptr(y), _ptr(ws), ws.numel(),
        _stream(x, offsets, sorted_rows, *ex.tensors(), ws)), "moe_expert_ffn")
    return y


def gate_up(x, offsets, sorted_rows, experts: PackedExperts, k: int = 4,
            h: Optional[torch.Tensor] = None) -> torch.Tensor:
    """-> h bf16 [T*k, 2880] (as int16 bits), SwiGLU of the gate/up projection
    of every routed slot, in expert-sorted order."""
    T = x.shape[0]
    ex = _experts(experts)
    E = ex.E
    _dev(x, "x", _BF16, (T, H))
    _dev(offsets, "offsets", _I32, (E + 1,))
    _dev(sorted_rows, "sorted_rows", _I32, (T * k,))
    if h is None:
        h = torch.empty((T * k, I), dtype=torch.int16, device=x.device)
    else:
        _dev(h, "h", _BF16, (T * k, I))
    _check(_native.lib().moe_gate_up(
        _ptr(x), _ptr(offsets), _ptr(sorted_rows), ex.w13.desc(), _ptr(ex.b13), T, E, k, _ptr(h),
        _stream(x, offsets, sorted_rows, ex.w13.codes, ex.w13.scales, ex.b13, h)), "moe_gate_up")
    return h


def gate_up_mx6(x_records, offsets, sorted_rows, experts: PackedExperts, k: int = 4,
                h: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gate_up with the activations as encode_mx6 records uint8 [T, 23, 256]."""
    T = x_records.shape[0]
    ex = _experts(experts)
    E = ex.E
    _dev(x_records, "x_records", _U8, (T, 23, 256))
    _dev(offsets, "offsets", _I32, (E + 1,))
    _dev(sorted_rows, "sorted_rows", _I32, (T * k,))
    if h is None:
        h = torch.empty((T * k, I), dtype=torch.int16, device=x_records.device)
    else:
        _dev(h, "h", _BF16, (T * k, I))
    _check(_native.lib().moe_gate_up_mx6(
        _ptr(x_records), _ptr(offsets), _ptr(sorted_rows), ex.w13.desc(), _ptr(ex.b13), T, E, k,
        _ptr(h), _stream(x_records, offsets, sorted_rows, ex.w13.codes, ex.w13.scales, ex.b13, h)),
        "moe_gate_up_mx6")
    return h


def down_accumulate(h, offsets, sorted_rows, topk_w, experts: PackedExperts,
                    out: torch.Tensor, k: int = 4) -> torch.Tensor:
    """out[t] += sum_j topk_w[t, j] * (W2[e] h + b2[e]) over the slots of t; returns out."""
    T = out.shape[0]
    ex = _experts(experts)
    E = ex.E
    _dev(out, "out", _F32, (T, H))
    _dev(h, "h", _BF16, (T * k, I))
    _dev(topk_w, "topk_w", _F32, (T, k))
    _dev(offsets, "offsets", _I32, (E + 1,))
    _dev(sorted_rows, "sorted_rows", _I32, (T * k,))
    _check(_native.lib().moe_down_accumulate(
        _ptr(h), _ptr(offsets), _ptr(sorted_rows), _ptr(topk_w), ex.w2.desc(), _ptr(ex.b2), T, E, k,
        _ptr(out), _stream(out, h, offsets, sorted_rows, topk_w, ex.w2.codes, ex.w2.scales, ex.b2)),
        "moe_down_accumulate")
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


def forward(x, Wr, br, experts: PackedExperts, k: int = 4, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer -> out fp32 [T, 2880]."""
    return _forward("moe_forward", "forward", x, Wr, br, experts, k, out, workspace)


def forward_mx6(x, Wr, br, experts: PackedExperts, k: int = 4,
                out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer with the tiled expert GEMMs on the block-scaled FP4 x FP6
    matrix cores (activations as two MX FP6 pieces) -> out fp32 [T, 2880]."""
    return _forward("moe_forward_mx6", "forward_mx6", x, Wr, br, experts, k, out, workspace)


def forward_noalloc(x, Wr, br, experts: PackedExperts, out: torch.Tensor,
                    k: int = 4) -> torch.Tensor:
    """The whole layer into the caller's out fp32 [T, 2880], with the library's
    own device scratch instead of a workspace: nothing is allocated, here or in
    the library (moe_forward_noalloc). Calls that overlap on one GPU race."""
    T = x.shape[0]
    E = Wr.shape[0]
    _dev(x, "x", _BF16, (T, H))
    _dev(Wr, "Wr", _F32, (E, H))
    _dev(br, "br", _F32, (E,))
    ex = _experts(experts, E)
    _dev(out, "out", _F32, (T, H))
    _check(_native.lib().moe_forward_noalloc(
        _ptr(x), _ptr(Wr), _ptr(br), ex.w13.desc(), _ptr(ex.b13), ex.w2.desc(), _ptr(ex.b2),
        T, E, k, _ptr(out), _stream(x, Wr, br, *ex.tensors(), out)), "moe_forward_noalloc")
    return out


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


def forward_block(x, norm_scale, Wr, br, experts: PackedExperts, k: int = 4,
                  norm_eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out fp32 [T, 2880] = x + layer(RMSNorm(x)): the MoE sublayer of a
    decoder layer with its pre-norm and residual add (the router takes the
    normed input in fp32, the expert GEMMs in bf16)."""
    T = x.shape[0]
    E = Wr.shape[0]
    _dev(x, "x", _BF16, (T, H))
    _dev(norm_scale, "norm_scale", _F32, (H,))
    _dev(Wr, "Wr", _F32, (E, H))
    _dev(br, "br", _F32, (E,))
    ex = _experts(experts, E)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    else:
        _dev(out, "out", _F32, (T, H))
    ws = _workspace(T, E, k, x.device, workspace, "forward_block")
    _check(_native.lib().moe_forward_block(
        _ptr(x), _ptr(norm_scale), float(norm_eps), _ptr(Wr), _ptr(br), ex.w13.desc(),
        _ptr(ex.b13), ex.w2.desc(), _ptr(ex.b2), T, E, k, _ptr(out), _ptr(ws), ws.numel(),
        _stream(x, norm_scale, Wr, br, *ex.tensors(), out, ws)), "moe_forward_block")
    return out


def _forward(fn, op, x, Wr, br, experts, k, out, workspace) -> torch.Tensor:
    T = x.shape[0]
    E = Wr.shape[0]
    _dev(x, "x", _BF16, (T, H))
    _dev(Wr, "Wr", _F32, (E, H))
    _dev(br, "br", _F32, (E,))
    ex = _experts(experts, E)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    else:
        _dev(out, "out", _F32, (T, H))
    ws = _workspace(T, E, k, x.device, workspace, op)
    _check(getattr(_native.lib(), fn)(
        _ptr(x), _ptr(Wr), _ptr(br), ex.w13.desc(), _ptr(ex.b13), ex.w2.desc(), _ptr(ex.b2),
        T, E, k, _ptr(out), _ptr(ws), ws.numel(), _stream(x, Wr, br, *ex.tensors(), out, ws)), fn)
    return out
