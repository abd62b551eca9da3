"""Plain fp64 CPU oracle of the gpt-oss mixture-of-experts FFN layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path (the HIP library and its Python binding) never touches it, and
this module imports nothing from the product path.

What it computes, step by step, each as its plain definition in float64:

* router logits ``x @ Wr^T + br`` -- gpt-oss-120b techniques map
  (models.inteligile.com), "Checked in its code" table, row "Auxiliary-loss-free
  load balancing": the router is a linear layer with a bias, giving one logit
  per (token, expert).
* top-k selection, k = experts_per_token = 4 -- same table, row "Mixture of
  experts" (a top-k over the router logits); "GPT-OSS 20B"/"GPT-OSS 120B" pages,
  raw config.json fields (experts_per_token, num_experts_per_tok).
  Reading: descending logit, equal logits ordered by lower expert index.
* routing weights = softmax over the k selected logits -- techniques map, same
  row as the router ("standard softmax top-k").
* expert-sorted permutation (counts, offsets, stable sorted rows) -- not on the
  pages; it is the grouping every grouped-GEMM MoE uses and is returned here
  so that the GPU permutation can be compared bit for bit.
* MXFP4 expert weights -- techniques map, "inference & serving" list
  ("MXFP4 weight quantization", "MXFP4 tensor packing"). The element and scale
  encodings are not printed on the pages; they follow the OCP Microscaling
  (MX) v1.0 formats: FP4 E2M1 elements, 32 elements share one E8M0 scale
  2^(s-127). Dequantisation here is a table lookup.
* SwiGLU with the gpt-oss clamp -- techniques map, row "SwiGLU feed-forward":
  ``glu = gate * sigmoid(gate * alpha)``, output ``(up + 1) * glu``; clamp
  limit swiglu_limit = 7 from the raw config.json fields. Readings: alpha =
  1.702 (named but not valued on the pages); gate clamped from above only, up
  clamped to [-7, 7], both after the bias; gate/up rows interleaved in w13
  (row 2i = gate i, row 2i+1 = up i).
* down projection with bias, and the routing-weighted sum of the k expert
  outputs -- the expert shapes (gate/up [2I, H] + bias, down [H, I] + bias,
  router [E, H] + bias) are the ones whose parameter count reproduces the
  checkpoint total printed on the "gpt-oss-20b" page (neurarch.com, "Our count
  against the checkpoint").

Layouts (row-major):
  x         [T, H]        uint16 bf16 bit patterns
  Wr        [E, H]        float32      br [E] float32
  w13_codes [E, 2I, H/2]  uint8: low nibble = even K index, high nibble = odd
  w13_scales[E, 2I, H/32] uint8: byte j scales K in [32j, 32j+31]
  b13       [E, 2I]       uint16 bf16 bits
  w2_codes  [E, H, I/2]   w2_scales [E, H, I/32]   b2 [E, H] bf16 bits
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

SWIGLU_ALPHA = 1.702
SWIGLU_LIMIT = 7.0

# FP4 E2M1 element values by 4-bit code (OCP MX v1.0): bit 3 is the sign,
# codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                       -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
                      dtype=np.float64)


def e8m0_scale(s: np.ndarray) -> np.ndarray:
    """E8M0 shared scale: byte s encodes 2^(s-127); s = 255 is NaN."""
    s = np.asarray(s)
    out = np.ldexp(1.0, s.astype(np.int64) - 127)
    return np.where(s == 255, np.nan, out)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 [..., N, K/2] codes + [..., N, K/32] scales -> float64 [..., N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = E2M1_TABLE[codes & 0x0F]
    hi = E2M1_TABLE[codes >> 4]
    K = codes.shape[-1] * 2
    vals = np.empty(codes.shape[:-1] + (K,), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    sc = e8m0_scale(scales)
    if sc.shape[-1] * 32 != K:
        raise ValueError("scale count does not match 32-element blocks")
    return vals * np.repeat(sc, 32, axis=-1)


def expert_parameter_shapes(H: int, I: int) -> Dict[str, tuple]:
    """Logical parameter shapes of one expert (gate/up, its bias, down, its bias)."""
    return {"w13": (2 * I, H), "b13": (2 * I,), "w2": (H, I), "b2": (H,)}


def router_parameter_shapes(H: int, E: int) -> Dict[str, tuple]:
    return {"Wr": (E, H), "br": (E,)}


def router_logits(x_bits: np.ndarray, Wr: np.ndarray, br: np.ndarray) -> np.ndarray:
    return router_logits_f64(bf16_to_f64(x_bits), Wr, br)


def router_logits_f64(x: np.ndarray, Wr: np.ndarray, br: np.ndarray) -> np.ndarray:
    """The router linear layer on float64 activations."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(Wr, dtype=np.float64).T + \
        np.asarray(br, dtype=np.float64)


def select_topk(logits: np.ndarray, k: int):
    """Indices of the k largest logits per row, descending, ties -> lower index.

    Also returns the gap between the k-th and (k+1)-th largest logit
    (inf when there are only k experts).
    """
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int64)
    srt = np.take_along_axis(logits, order, axis=1)
    gap = (srt[:, k - 1] - srt[:, k]) if E > k else np.full(T, np.inf)
    return ids, gap


def routing_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits of each token."""
    sel = np.take_along_axis(logits, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def expert_permutation(ids: np.ndarray, E: int):
    """Group the T*k routed slots by expert, keeping slot order within an expert.

    Returns counts [E], offsets [E+1] and sorted_rows [T*k], whose entries are
    flat slot indices t*k + j.
    """
    flat = np.asarray(ids).reshape(-1)
    sorted_rows = np.argsort(flat, kind="stable").astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets, sorted_rows


def swiglu(gu: np.ndarray, alpha: float = SWIGLU_ALPHA,
           limit: float = SWIGLU_LIMIT) -> np.ndarray:
    """gpt-oss gated unit on interleaved gate/up columns."""
    gate = np.minimum(gu[..., 0::2], limit)
    up = np.clip(gu[..., 1::2], -limit, limit)
    # exp overflows to inf for very negative gates; gate / inf is the correct limit 0
    with np.errstate(over="ignore"):
        glu = gate / (1.0 + np.exp(-alpha * gate))
    return (up + 1.0) * glu


def expert_mlp(xe: np.ndarray, W13: np.ndarray, b13: np.ndarray,
               W2: np.ndarray, b2: np.ndarray, alpha: float = SWIGLU_ALPHA,
               limit: float = SWIGLU_LIMIT) -> np.ndarray:
    """One expert on rows xe [n, H]: gate/up projection, SwiGLU, down projection."""
    gu = xe @ W13.T + b13
    h = swiglu(gu, alpha, limit)
    return h @ W2.T + b2


def expert_weights(inputs: Dict[str, np.ndarray], e: int):
    """Dequantised float64 weights and biases of expert e."""
    W13 = dequant_mxfp4(inputs["w13_codes"][e], inputs["w13_scales"][e])
    W2 = dequant_mxfp4(inputs["w2_codes"][e], inputs["w2_scales"][e])
    return W13, bf16_to_f64(inputs["b13"][e]), W2, bf16_to_f64(inputs["b2"][e])


def route(inputs: Dict[str, np.ndarray], k: int):
    logits = router_logits(inputs["x"], inputs["Wr"], inputs["br"])
    ids, gap = select_topk(logits, k)
    w = routing_weights(logits, ids)
    return logits, ids, w, gap


def forward(inputs: Dict[str, np.ndarray], k: int,
            tokens: Optional[Sequence[int]] = None,
            ids_override: Optional[np.ndarray] = None,
            alpha: float = SWIGLU_ALPHA, limit: float = SWIGLU_LIMIT,
            keep_y: bool = False,
            router_x: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The whole layer in float64.

    ``router_x`` (float64 [T, H]), when given, is what the router sees in
    place of the bf16 ``x``; the experts still take ``x`` (the decoder block
    routes on its unrounded normed input, oracle/block.py).

    ``tokens`` restricts the expert computation to those token indices (the
    routing is still computed for every token); ``ids_override`` [T, k]
    replaces the selected experts of every token (weights are then the softmax
    of the float64 logits of the given experts). Only experts that some
    computed token selects are dequantised, one at a time.
    """
    if router_x is None:
        logits = router_logits(inputs["x"], inputs["Wr"], inputs["br"])
    else:
        logits = router_logits_f64(router_x, inputs["Wr"], inputs["br"])
    T, E = logits.shape
    ids, gap = select_topk(logits, k)
    if ids_override is not None:
        ids = np.asarray(ids_override, dtype=np.int64).reshape(T, k)
    w = routing_weights(logits, ids)
    counts, offsets, sorted_rows = expert_permutation(ids, E)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    x = bf16_to_f64(inputs["x"][tok])
    H = x.shape[1]
    out = np.zeros((tok.size, H), dtype=np.float64)
    y = np.zeros((tok.size, k, H), dtype=np.float64) if keep_y else None
    sel = ids[tok]
    for e in np.unique(sel):
        rows, slots = np.nonzero(sel == e)
        W13, b13, W2, b2 = expert_weights(inputs, int(e))
        ye = expert_mlp(x[rows], W13, b13, W2, b2, alpha, limit)
        out[rows] += w[tok[rows], slots][:, None] * ye
        if keep_y:
            y[rows, slots] = ye
    res = dict(logits=logits, ids=ids, w=w, gap=gap, counts=counts,
               offsets=offsets, sorted_rows=sorted_rows, tokens=tok, out=out)
    if keep_y:
        res["y"] = y
    return res
