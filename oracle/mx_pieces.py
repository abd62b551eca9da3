"""MX block quantisation of activations into two FP6 E2M3 pieces.

TEST INFRASTRUCTURE, under the same rules as ``oracle.moe_oracle``: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import it; the product path never does, and this module imports
nothing from it.

The pages fix MXFP4 for the expert weights ("gpt-oss-120b" techniques map,
"inference & serving": MXFP4 weight quantization). Block-scaled matrix cores
take both operands as MX blocks, so an activation row can be fed to them as
a short sum of MX blocks. This module is the definition of that encoding,
written from the OCP Microscaling Formats (MX) v1.0 specification (not on
the pages):

* FP6 E2M3 element: sign bit 5, exponent bits 4..3 (bias 1), mantissa bits
  2..0; exponent field 0 is subnormal (m/8). Largest magnitude 7.5, no
  Inf/NaN. emax_elem = 2.
* Conversion of a block V of 32 values (MX v1.0, "conversion from a vector of
  scalars"): shared exponent X = floor(log2(max|V_i|)) - emax_elem, element
  P_i = V_i / 2^X rounded to the nearest E2M3 value, ties to the even
  mantissa, magnitudes past 7.5 clamped to 7.5. Scale byte = X + 127.
* Two pieces: P1 encodes V; P2 encodes the exact residual V - dequant(P1).
  The pair stands for dequant(P1) + dequant(P2).

Readings where the specification leaves a choice (the HIP encoder makes the
same ones): an all-zero block gets X = 0 (scale byte 127) and zero codes; X is
clamped to [-127, 127]; the sign bit is set exactly for negative inputs (a
negative value that rounds to zero is encoded as -0).
"""
from __future__ import annotations

import numpy as np

E2M3_EMAX = 2
E2M3_MAX = 7.5


def e2m3_value(code: np.ndarray) -> np.ndarray:
    """FP6 E2M3 code (0..63) -> float64 value."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x20, -1.0, 1.0)
    e = (c >> 3) & 0x3
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * np.ldexp(1.0, e - 1))
    return sign * mag


# magnitudes of codes 0..31, increasing with the code
_E2M3_MAGS = e2m3_value(np.arange(32))


def shared_exponent(block_absmax: np.ndarray) -> np.ndarray:
    """X = floor(log2(amax)) - emax_elem, clamped to [-127, 127]; 0 for amax 0."""
    a = np.asarray(block_absmax, dtype=np.float64)
    _, e = np.frexp(np.where(a > 0, a, 1.0))   # a = f * 2^e, f in [0.5, 1)
    X = (e - 1) - E2M3_EMAX
    X = np.where(a > 0, X, 0)
    return np.clip(X, -127, 127).astype(np.int64)


def e2m3_round(a: np.ndarray) -> np.ndarray:
    """Magnitude code (0..31) nearest to a >= 0 on the E2M3 grid, ties to the
    even code, saturating at 7.5."""
    a = np.minimum(np.asarray(a, dtype=np.float64), E2M3_MAX)
    hi = np.searchsorted(_E2M3_MAGS, a, side="left")      # first grid value >= a
    hi = np.clip(hi, 0, 31)
    lo = np.clip(hi - 1, 0, 31)
    d_lo = a - _E2M3_MAGS[lo]
    d_hi = _E2M3_MAGS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo)


def mx_e2m3_quantize(v: np.ndarray):
    """One MX E2M3 piece of v [..., 32*nb]: codes [..., nb, 32] (0..63) and
    scale bytes [..., nb]."""
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(v.shape[:-1] + (-1, 32))
    X = shared_exponent(np.abs(blocks).max(axis=-1))
    scaled = blocks / np.ldexp(1.0, X)[..., None]
    mag = e2m3_round(np.abs(scaled))
    codes = mag + np.where(scaled < 0, 32, 0)
    return codes.astype(np.uint8), (X + 127).astype(np.uint8)


def mx_e2m3_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [..., nb, 32], scale bytes [..., nb] -> float64 [..., 32*nb]."""
    vals = e2m3_value(codes) * np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    return vals.reshape(vals.shape[:-2] + (-1,))


def mx6x2_pieces(v: np.ndarray):
    """Two-piece encoding of v [..., 32*nb]: (codes1, scales1, codes2, scales2)."""
    v = np.asarray(v, dtype=np.float64)
    c1, s1 = mx_e2m3_quantize(v)
    r = v - mx_e2m3_dequant(c1, s1)
    c2, s2 = mx_e2m3_quantize(r)
    return c1, s1, c2, s2


def mx6x2_value(v: np.ndarray) -> np.ndarray:
    """What the two pieces of v stand for: dequant(P1) + dequant(P2)."""
    c1, s1, c2, s2 = mx6x2_pieces(v)
    return mx_e2m3_dequant(c1, s1) + mx_e2m3_dequant(c2, s2)
