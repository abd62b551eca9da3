"""The RMSNorm + residual neighbours of the oracle against their pins (no GPU),
and two plausible routing mistakes planted in the block oracle that the pins
must catch."""
import numpy as np
import pytest

import oracle.block as ob
import oracle.moe_oracle as om
from tests.block_pins import ALL_CHECKS

_real_forward = om.forward


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_block_pin(check):
    check()


def _routes_on_bf16_norm(inputs, k, **kw):
    kw.pop("router_x", None)
    return _real_forward(inputs, k, **kw)


def _routes_on_raw_input(x_bits):
    def fwd(inputs, k, **kw):
        kw["router_x"] = om.bf16_to_f64(x_bits)
        return _real_forward(inputs, k, **kw)
    return fwd


def _failed_checks():
    failed = []
    for check in ALL_CHECKS:
        try:
            check()
        except Exception:  # an exception of any kind means the pin caught it
            failed.append(check.__name__)
    return failed


def test_mutation_router_on_rounded_norm(monkeypatch):
    monkeypatch.setattr(om, "forward", _routes_on_bf16_norm)
    assert "check_block_routes_on_unrounded_norm" in _failed_checks()


def test_mutation_router_on_unnormed_input(monkeypatch):
    real_block = ob.block_forward

    def block(inputs, k, scale, *a, **kw):
        monkeypatch.setattr(om, "forward", _routes_on_raw_input(inputs["x"]))
        try:
            return real_block(inputs, k, scale, *a, **kw)
        finally:
            monkeypatch.setattr(om, "forward", _real_forward)

    monkeypatch.setattr(ob, "block_forward", block)
    assert _failed_checks()
