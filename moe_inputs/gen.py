"""Seeded synthetic inputs with the shapes and value distributions of the
gpt-oss MoE FFN layer.

Shapes follow the config fields printed on the model pages ("GPT-OSS 20B",
raw config.json fields table; "GPT-OSS 120B", config.json full-fields table):
hidden_size = intermediate_size = 2880, num_local_experts = 32 (20b) or 128
(120b), experts_per_token = 4.

Value recipe (one ``numpy.random.Generator(PCG64(seed))`` per input set, draws
in this fixed order):

1. x      bf16 [T, H]      N(0, 1), rounded to nearest even
2. Wr     fp32 [E, H]      N(0, 0.02)
3. br     fp32 [E]         N(0, 0.02), or a calibrated Zipf bias (below)
4. w13 code bytes  u8 [E, 2I, H/2]   uniform bytes: both nibbles uniform over 16 codes
5. w13 scale bytes u8 [E, 2I, H/32]  127 + U{-8..-5}
6. b13    bf16 [E, 2I]     N(0, 0.02)
7. w2 code bytes   u8 [E, H, I/2]
8. w2 scale bytes  u8 [E, H, I/32]
9. b2     bf16 [E, H]      N(0, 0.02)

Zipf-skewed routing (the 120b configurations): the pages give no load
distribution. The target share of expert rank r is proportional to r^-s,
capped at 1/k (an expert can take at most one of a token's k slots) with the
excess water-filled over the uncapped ranks; ranks map to expert ids through a
seeded permutation. The router bias is fitted to that target on *stand-in*
logits: independent Gaussians with the router rows' norms as standard
deviations (a token's logits x.Wr[e] are close to independent N(0, |Wr[e]|^2)
for x ~ N(0, I)). The fit never sees the actual x, so it shares no arithmetic
with the layer; it only shapes the input distribution, and the realised load
is whatever the layer computes from it.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

H_DEFAULT = 2880
I_DEFAULT = 2880


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    E: int
    k: int
    zipf_s: Optional[float]
    regime: str  # "decode" (weight-streaming) or "prefill" (matrix-core bound)
    note: str


LAYER_CONFIGS = [
    LayerConfig("gpt-oss-20b T=16", 16, 32, 4, None, "decode",
                "20b layer, 16 tokens; the small case the oracle finishes in seconds"),
    LayerConfig("gpt-oss-20b decode T=64", 64, 32, 4, None, "decode",
                "20b layer, decode batch of 64 tokens; bound by MXFP4 weight bytes"),
    LayerConfig("gpt-oss-20b prefill T=4096", 4096, 32, 4, None, "prefill",
                "20b layer, 4096-token prefill (the initial context length)"),
    LayerConfig("gpt-oss-120b T=8192 zipf1.1", 8192, 128, 4, 1.1, "prefill",
                "120b layer, 8192 tokens, Zipf(1.1) expert load"),
    LayerConfig("gpt-oss-120b mixed T=16384 zipf1.3", 16384, 128, 4, 1.3, "prefill",
                "120b layer, 256 decode + 16128 prefill tokens in one call, Zipf(1.3) load"),
]


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bit patterns, round to nearest even.

    Input encoding only (finite inputs): the layer never calls this.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def zipf_target_shares(E: int, k: int, s: float) -> np.ndarray:
    """Per-rank target share of the T*k routed slots: r^-s, capped at 1/k.

    The cap is applied by water-filling: capped ranks hold exactly 1/k and the
    remaining mass is spread over the others in proportion to r^-s.
    """
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    cap = 1.0 / k
    capped = np.zeros(E, dtype=bool)
    shares = p.copy()
    for _ in range(E):
        over = (shares > cap * (1 + 1e-12)) & ~capped
        if not over.any():
            break
        capped |= over
        rest = ~capped
        shares[capped] = cap
        shares[rest] = p[rest] / p[rest].sum() * (1.0 - cap * capped.sum())
    return shares


def _fit_zipf_bias(row_norms: np.ndarray, k: int, s: float,
                   rng: np.random.Generator, n_sim: int = 8192,
                   iters: int = 200) -> np.ndarray:
    """Fit a router bias so that top-k selection on stand-in logits follows
    the capped Zipf target (see module docstring)."""
    E = row_norms.shape[0]
    shares = zipf_target_shares(E, k, s)
    perm = rng.permutation(E)              # rank r -> expert perm[r]
    target = np.empty(E)
    target[perm] = shares * k              # selection probability per token
    z = rng.standard_normal((n_sim, E)) * row_norms[None, :]
    b = np.zeros(E)
    floor = 0.25 / n_sim
    for _ in range(iters):
        part = np.argpartition(-(z + b[None, :]), k - 1, axis=1)[:, :k]
        realised = np.bincount(part.ravel(), minlength=E) / n_sim
        b += 0.5 * (np.log(np.maximum(target, floor))
                    - np.log(np.maximum(realised, floor)))
        b -= b.mean()
    return b.astype(np.float32)


def _uniform_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def make_layer_inputs(T: int, E: int, k: int, seed: int = 0,
                      zipf_s: Optional[float] = None,
                      H: int = H_DEFAULT, I: int = I_DEFAULT,
                      scale_exp_range=(-8, -5),
                      router_only: bool = False) -> Dict[str, np.ndarray]:
    """Draw one input set of the layer. Returns host arrays:

    x [T,H] u16 (bf16 bits), Wr [E,H] f32, br [E] f32,
    w13_codes [E,2I,H/2] u8, w13_scales [E,2I,H/32] u8, b13 [E,2I] u16,
    w2_codes [E,H,I/2] u8, w2_scales [E,H,I/32] u8, b2 [E,H] u16.
    ``router_only`` stops after the router inputs (x, Wr, br); the draws of
    those three are the same as in the full set.
    """
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of the 32-element MX block")
    rng = np.random.Generator(np.random.PCG64(seed))
    lo, hi = scale_exp_range
    x = bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    Wr = (rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    br = (rng.standard_normal(E, dtype=np.float32) * np.float32(0.02))
    if zipf_s is not None:
        zrng = np.random.Generator(np.random.PCG64([seed, 0x5A1F]))
        norms = np.sqrt((Wr.astype(np.float64) ** 2).sum(axis=1))
        br = _fit_zipf_bias(norms, k, zipf_s, zrng)
    if router_only:
        return dict(x=x, Wr=Wr, br=br)
    w13_codes = _uniform_bytes(rng, (E, 2 * I, H // 2))
    w13_scales = (127 + rng.integers(lo, hi + 1, size=(E, 2 * I, H // 32))).astype(np.uint8)
    b13 = bf16_bits_from_f32(rng.standard_normal((E, 2 * I), dtype=np.float32) * np.float32(0.02))
    w2_codes = _uniform_bytes(rng, (E, H, I // 2))
    w2_scales = (127 + rng.integers(lo, hi + 1, size=(E, H, I // 32))).astype(np.uint8)
    b2 = bf16_bits_from_f32(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    return dict(x=x, Wr=Wr, br=br, w13_codes=w13_codes, w13_scales=w13_scales,
                b13=b13, w2_codes=w2_codes, w2_scales=w2_scales, b2=b2)


def make_config_inputs(index: int, seed: int = 0, router_only: bool = False) -> Dict[str, np.ndarray]:
    c = LAYER_CONFIGS[index]
    return make_layer_inputs(c.T, c.E, c.k, seed=seed, zipf_s=c.zipf_s, router_only=router_only)


def device_activations(T: int, seed: int = 0, H: int = H_DEFAULT, device="cuda"):
    """x [T, H] as bf16 bit patterns (int16 tensor) drawn on the device: float32
    N(0, 1) from torch's generator for that device seeded with ``seed``,
    rounded to bf16 (nearest even). The distribution of ``make_layer_inputs``'
    x, for row counts whose host draw would take minutes; the values differ
    from the host draw. Read rows back to the host for the oracle."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    chunk = 1 << 16
    for r0 in range(0, T, chunk):
        n = min(chunk, T - r0)
        x[r0:r0 + n] = torch.randn((n, H), generator=g, device=device,
                                   dtype=torch.float32).to(torch.bfloat16)
    return x.view(torch.int16)
