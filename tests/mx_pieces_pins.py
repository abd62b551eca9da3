"""Pins of the two-piece MX E2M3 activation encoding (oracle/mx_pieces.py)
against routes that do not use its helpers: the E2M3 bit fields decoded in a
Python loop, nearest-value search by enumerating the whole grid, exact
round trips of every code, and the error bound the construction implies.
The definition itself is the OCP Microscaling Formats v1.0 conversion of a
32-value block to FP6 E2M3."""
from __future__ import annotations

import numpy as np

import oracle.mx_pieces as mp


def e2m3_from_bits(c: int) -> float:
    """FP6 E2M3: sign bit 5, exponent bits 4..3 (bias 1), mantissa bits 2..0."""
    sign = -1.0 if c & 0x20 else 1.0
    e = (c >> 3) & 0x3
    m = c & 0x7
    if e == 0:
        return sign * m * 0.125
    return sign * (1.0 + m * 0.125) * 2.0 ** (e - 1)


def nearest_code_by_search(a: float) -> int:
    """Magnitude code nearest to a (>= 0) by trying all 32; ties -> even code;
    anything past the largest value takes the largest."""
    best, best_d = 0, None
    for c in range(32):
        d = abs(e2m3_from_bits(c) - min(a, 7.5))
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def check_e2m3_table():
    for c in range(64):
        assert mp.e2m3_value(c) == e2m3_from_bits(c), c
    mags = sorted({abs(e2m3_from_bits(c)) for c in range(64)})
    assert len(mags) == 32 and mags[0] == 0.0 and mags[-1] == 7.5
    assert e2m3_from_bits(0b001000) == 1.0 and e2m3_from_bits(0b000001) == 0.125
    assert e2m3_from_bits(0b111111) == -7.5


def check_rounding_by_search():
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.uniform(0, 8, 3000), rng.uniform(0, 1, 1000),
                        np.arange(0, 8.01, 1 / 32)])
    got = mp.e2m3_round(a)
    for ai, gi in zip(a, got):
        assert gi == nearest_code_by_search(float(ai)), (ai, gi)


def check_ties_to_even():
    for c in range(31):
        mid = 0.5 * (e2m3_from_bits(c) + e2m3_from_bits(c + 1))
        want = c if c % 2 == 0 else c + 1
        assert mp.e2m3_round(np.array([mid]))[0] == want, (c, mid)


def check_round_trip_every_code():
    for X in (-20, -3, 0, 7):
        for c in range(64):
            block = np.zeros(32)
            block[0] = 4.0 * 2.0 ** X            # fixes the shared exponent at X
            block[5] = e2m3_from_bits(c) * 2.0 ** X
            codes, scales = mp.mx_e2m3_quantize(block)
            assert scales[0] == X + 127
            want = 0 if c == 32 else c            # -0.0 is not negative: +0
            assert codes[0, 5] == want, (X, c, codes[0, 5])
            assert codes[0, 0] == 0b011000      # 4.0 = exponent field 3, mantissa 0


def check_shared_exponent_and_saturation():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((200, 32)) * np.ldexp(1.0, rng.integers(-30, 30, (200, 1)))
    codes, scales = mp.mx_e2m3_quantize(v)
    amax = np.abs(v).max(axis=1)
    ratio = amax / np.ldexp(1.0, scales.astype(np.int64)[:, 0] - 127)
    assert np.all((ratio >= 4.0) & (ratio < 8.0))
    z_codes, z_scales = mp.mx_e2m3_quantize(np.zeros(32))
    assert z_scales[0] == 127 and not z_codes.any()
    sat = np.zeros(32)
    sat[3], sat[4] = 7.8, -7.9
    codes, scales = mp.mx_e2m3_quantize(sat)
    assert scales[0] == 127 and codes[0, 3] == 31 and codes[0, 4] == 63


def check_two_piece_error_bound():
    """|v - (P1 + P2)| <= amax(block) / 256: the residual is at most a quarter
    of the first scale, so the second scale is at least 16x finer, and the
    second rounding is within a quarter of that scale."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 2880)) * np.exp(rng.uniform(-3, 3, (64, 1)))
    v = v.astype(np.float32).astype(np.float64)
    approx = mp.mx6x2_value(v)
    blocks = np.abs(v).reshape(64, 90, 32).max(axis=-1)
    err = np.abs(v - approx).reshape(64, 90, 32).max(axis=-1)
    assert np.all(err <= blocks / 256.0)
    # a block that one piece already holds exactly leaves a zero second piece
    exact = np.array([e2m3_from_bits(c) for c in range(32)]) * 0.25
    c1, s1, c2, s2 = mp.mx6x2_pieces(exact)
    assert not c2.any() and s2[0] == 127
    assert np.array_equal(mp.mx_e2m3_dequant(c1, s1), exact)


ALL_CHECKS = [check_e2m3_table, check_rounding_by_search, check_ties_to_even,
              check_round_trip_every_code, check_shared_exponent_and_saturation,
              check_two_piece_error_bound]
