"""The MoE layer with its two neighbours in the decoder block: the pre-MoE
RMSNorm and the residual add.

TEST INFRASTRUCTURE, under the same rules as ``oracle.moe_oracle``: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import it; the product path never does.

  t   = RMSNorm(x) = x / sqrt(mean(x^2) + eps) * scale     (per token, over H)
  out = x + MoE(t), the router on t, the experts on bf16(t)

Sources: the "gpt-oss-20b" page (neurarch.com), "Structure" table: every
decoder layer runs RMSNorm_i_2 -> MoE_i -> Add_i_ffn, i.e. the MoE sees the
normed hidden state and its output is added to the un-normed one; the
"gpt-oss-120b" techniques map, "normalization & residual" (RMSNorm, Pre-LN);
the GPT-OSS 20B / 120B raw config.json tables (rms_norm_eps = 1e-5).
Readings where the pages are silent: RMSNorm is the textbook
x / sqrt(mean(x^2) + eps) * scale with a float32 scale vector of H values;
the router, a float32 linear layer with float32 weights, takes the normed
activations as they are (unrounded; float64 here); the expert GEMMs take them
rounded once to bf16 (round to nearest even), their matrix-core input type,
as they take h; the residual is the bf16 block input x, added in float to the
float32 layer output.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import moe_oracle as om

RMS_NORM_EPS = 1e-5


def rmsnorm(x_bits: np.ndarray, scale: np.ndarray, eps: float = RMS_NORM_EPS) -> np.ndarray:
    """Per row: x / sqrt(mean(x^2) + eps) * scale, in float64."""
    x = om.bf16_to_f64(x_bits)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(scale, dtype=np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, one rounding to nearest even (finite
    values in the normal bf16 range, or zero)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    b = v.view(np.uint64)
    sign = (b >> np.uint64(63)).astype(np.uint64)
    mag = b & np.uint64(0x7FFFFFFFFFFFFFFF)
    # keep 7 of the 52 mantissa bits: round the dropped 45 bits to nearest even
    keep = (mag >> np.uint64(45)) & np.uint64(1)
    r = (mag + np.uint64((1 << 44) - 1) + keep) >> np.uint64(45)   # exponent(11) | mantissa(7)
    exp64 = (r >> np.uint64(7)).astype(np.int64)
    mant = (r & np.uint64(0x7F)).astype(np.int64)
    exp16 = np.where(mag == 0, 0, exp64 - 1023 + 127)
    mant = np.where(mag == 0, 0, mant)
    if np.any((mag != 0) & ((exp16 <= 0) | (exp16 >= 255))):
        raise ValueError("value outside the normal bf16 range")
    return ((sign.astype(np.int64) << 15) | (exp16 << 7) | mant).astype(np.uint16)


def normed_input_bits(x_bits: np.ndarray, scale: np.ndarray,
                      eps: float = RMS_NORM_EPS) -> np.ndarray:
    """bf16(RMSNorm(x)): the activations the expert GEMMs see."""
    return f64_to_bf16_bits(rmsnorm(x_bits, scale, eps))


def block_forward(inputs: Dict[str, np.ndarray], k: int, scale: np.ndarray,
                  eps: float = RMS_NORM_EPS,
                  tokens: Optional[Sequence[int]] = None,
                  ids_override: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """out = x + MoE(RMSNorm(x)) in float64, routed on the normed input and
    with bf16(RMSNorm(x)) into the experts; also returns that bf16 input
    ("t") and everything ``moe_oracle.forward`` returns for it."""
    t = rmsnorm(inputs["x"], scale, eps)
    t_bits = f64_to_bf16_bits(t)
    res = om.forward(dict(inputs, x=t_bits), k, tokens=tokens, ids_override=ids_override,
                     router_x=t)
    res["out"] = res["out"] + om.bf16_to_f64(inputs["x"][res["tokens"]])
    res["t"] = t_bits
    return res
