"""The two-piece MX E2M3 encoding of the oracle against its pins (no GPU),
and planted mistakes that the pins must catch."""
import numpy as np
import pytest

import oracle.mx_pieces as mp
from tests.mx_pieces_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_mx_pieces_pin(check):
    check()


_real_round = mp.e2m3_round
_real_exp = mp.shared_exponent
_real_value = mp.e2m3_value


def _round_ties_up(a):
    a = np.minimum(np.asarray(a, dtype=np.float64), mp.E2M3_MAX)
    hi = np.clip(np.searchsorted(mp._E2M3_MAGS, a, side="left"), 0, 31)
    lo = np.clip(hi - 1, 0, 31)
    return np.where(mp._E2M3_MAGS[hi] - a <= a - mp._E2M3_MAGS[lo], hi, lo)


def _round_no_saturation(a):
    a = np.asarray(a, dtype=np.float64)
    return np.where(a > 7.5, 32, _real_round(a))   # overflows into the sign bit


def _exp_emax3(amax):
    return _real_exp(amax) - 1


def _exp_ceil(amax):
    a = np.asarray(amax, dtype=np.float64)
    return np.where(a > 0, np.ceil(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64) - 2, 0)


def _value_bias0(code):
    c = np.asarray(code, dtype=np.int64)
    return _real_value(c) * np.where(((c >> 3) & 3) == 0, 1.0, 2.0)


MUTATIONS = {
    "ties_away_from_zero": ("e2m3_round", _round_ties_up),
    "no_saturation": ("e2m3_round", _round_no_saturation),
    "emax_3": ("shared_exponent", _exp_emax3),
    "ceil_log2": ("shared_exponent", _exp_ceil),
    "exponent_bias_0": ("e2m3_value", _value_bias0),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mx_pieces_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mp, attr, fn)
    if attr == "e2m3_value":
        monkeypatch.setattr(mp, "_E2M3_MAGS", fn(np.arange(32)))
    failed = []
    for check in ALL_CHECKS:
        try:
            check()
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"mutation {name} passed every pin"
