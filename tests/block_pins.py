"""Pins of the RMSNorm + residual neighbours of the layer (oracle/block.py)
against routes that do not use its helpers: pure-Python loops, closed forms
for constant rows, exact power-of-two invariance, and the fp32 -> bf16
rounding of the input generator on values both routes must round alike."""
from __future__ import annotations

import math

import numpy as np

import oracle.block as ob
import oracle.moe_oracle as om
from moe_inputs import bf16_bits_from_f32, make_layer_inputs


def check_rmsnorm_python_loop():
    rng = np.random.default_rng(1)
    x = bf16_bits_from_f32(rng.standard_normal((3, 64)).astype(np.float32))
    g = rng.uniform(0.5, 1.5, 64)
    got = ob.rmsnorm(x, g, 1e-5)
    for r in range(3):
        vals = [om.bf16_to_f64(x[r:r + 1, c:c + 1])[0, 0] for c in range(64)]
        ms = sum(v * v for v in vals) / 64
        for c in range(64):
            assert abs(got[r, c] - vals[c] / math.sqrt(ms + 1e-5) * g[c]) < 1e-13


def check_rmsnorm_constant_rows():
    # a row of one value c: c / sqrt(c^2 + eps) * g, whatever the width
    for c in (3.0, -0.25, 1e-3):
        x = bf16_bits_from_f32(np.full((1, 2880), c, np.float32))
        cv = om.bf16_to_f64(x)[0, 0]
        got = ob.rmsnorm(x, np.full(2880, 2.0), 1e-5)
        assert np.allclose(got, 2.0 * cv / math.sqrt(cv * cv + 1e-5), rtol=1e-14, atol=0)
    zero = ob.rmsnorm(np.zeros((1, 2880), np.uint16), np.ones(2880), 1e-5)
    assert not zero.any()


def check_rmsnorm_scale_invariance():
    # eps = 0: scaling a row by 2^j (exact in bf16) leaves the result unchanged,
    # and the output has RMS exactly 1 up to rounding when scale = 1
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 2880)).astype(np.float32)
    a = ob.rmsnorm(bf16_bits_from_f32(x), np.ones(2880), 0.0)
    b = ob.rmsnorm(bf16_bits_from_f32(x * 8.0), np.ones(2880), 0.0)
    assert np.array_equal(a, b)
    assert np.allclose(np.sqrt(np.mean(a * a, axis=1)), 1.0, rtol=1e-13)


def check_bf16_rounding():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    v[:3] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)]   # ties -> even mantissa
    assert np.array_equal(ob.f64_to_bf16_bits(v.astype(np.float64)), bf16_bits_from_f32(v))
    assert ob.f64_to_bf16_bits(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert ob.f64_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82
    # one rounding from float64, not two: just above a tie rounds up
    assert ob.f64_to_bf16_bits(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81


def check_block_residual_and_zero_experts():
    """Zero expert codes: out = x + sum_j w_j b2[e_j], with the routing of the
    normed input."""
    T, E, k = 12, 8, 2
    inp = make_layer_inputs(T, E, k, seed=9)
    inp["w13_codes"][:] = 0
    inp["w2_codes"][:] = 0
    g = np.random.default_rng(4).uniform(0.5, 2.0, 2880)
    res = ob.block_forward(inp, k, g)
    t = ob.rmsnorm(inp["x"], g)   # the router sees the unrounded normed input
    logits = t @ inp["Wr"].astype(np.float64).T + inp["br"].astype(np.float64)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    z = np.exp(np.take_along_axis(logits, ids, 1) - np.take_along_axis(logits, ids, 1)[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    want = om.bf16_to_f64(inp["x"]) + np.einsum("tj,tjh->th", w, om.bf16_to_f64(inp["b2"])[ids])
    assert np.allclose(res["out"], want, rtol=1e-12, atol=1e-12)


def check_block_routes_on_unrounded_norm():
    """A constant row of ones normalises to 1/sqrt(1 + eps) = 0.999995, which
    bf16 rounds to 1.0. Expert 0 scores the row's mean, expert 1 a constant
    0.9999975 between the two: routing on the unrounded value picks expert 1,
    on the bf16 value expert 0. The expert part is zero (zero codes, zero
    biases), so out = x + b2 of the chosen expert exactly."""
    inp = make_layer_inputs(1, 2, 1, seed=11)
    inp["x"] = bf16_bits_from_f32(np.ones((1, 2880), np.float32))
    inp["Wr"] = np.zeros((2, 2880), np.float32)
    inp["Wr"][0, :] = np.float32(1.0 / 2880.0)
    inp["br"] = np.array([0.0, 0.9999975], np.float32)
    for key in ("w13_codes", "w2_codes", "b13"):
        inp[key][:] = 0
    inp["b2"][0, :] = bf16_bits_from_f32(np.full(2880, 3.0, np.float32))
    inp["b2"][1, :] = bf16_bits_from_f32(np.full(2880, -5.0, np.float32))
    res = ob.block_forward(inp, 1, np.ones(2880), 1e-5)
    wr0 = float(np.float32(1.0 / 2880.0)) * 2880.0   # expert 0's logit per unit input
    assert wr0 / math.sqrt(1.0 + 1e-5) < 0.9999975 < wr0   # the two routes disagree
    assert ob.normed_input_bits(inp["x"], np.ones(2880))[0, 0] == 0x3F80   # bf16(t) = 1.0
    assert int(res["ids"][0, 0]) == 1
    assert np.array_equal(res["out"], np.full((1, 2880), 1.0 - 5.0))


ALL_CHECKS = [check_rmsnorm_python_loop, check_rmsnorm_constant_rows,
              check_rmsnorm_scale_invariance, check_bf16_rounding,
              check_block_residual_and_zero_experts, check_block_routes_on_unrounded_norm]
