"""Plant plausible mistakes in the oracle (on the CPU) and show that the pins
catch every one of them. Each mutation replaces one oracle function or table
through monkeypatch; the real oracle is untouched afterwards."""
import numpy as np
import pytest

import oracle.moe_oracle as om
from tests.oracle_pins import ALL_CHECKS

_real_dequant = om.dequant_mxfp4
_real_swiglu = om.swiglu
_real_mlp = om.expert_mlp
_real_perm = om.expert_permutation


def _dequant_swapped_nibbles(codes, scales):
    c = np.asarray(codes, dtype=np.uint8)
    return _real_dequant(((c & 0xF) << 4) | (c >> 4), scales)


def _dequant_wrong_block(codes, scales):
    return _real_dequant(codes, np.roll(scales, 1, axis=-1))


def _swiglu_swapped(gu, alpha=om.SWIGLU_ALPHA, limit=om.SWIGLU_LIMIT):
    s = np.empty_like(gu)
    s[..., 0::2], s[..., 1::2] = gu[..., 1::2], gu[..., 0::2]
    return _real_swiglu(s, alpha, limit)


def _swiglu_no_plus_one(gu, alpha=om.SWIGLU_ALPHA, limit=om.SWIGLU_LIMIT):
    gate = np.minimum(gu[..., 0::2], limit)
    up = np.clip(gu[..., 1::2], -limit, limit)
    return up * gate / (1.0 + np.exp(-alpha * gate))


def _swiglu_two_sided_gate(gu, alpha=om.SWIGLU_ALPHA, limit=om.SWIGLU_LIMIT):
    gate = np.clip(gu[..., 0::2], -limit, limit)
    up = np.clip(gu[..., 1::2], -limit, limit)
    return (up + 1.0) * gate / (1.0 + np.exp(-alpha * gate))


def _swiglu_no_up_clamp(gu, alpha=om.SWIGLU_ALPHA, limit=om.SWIGLU_LIMIT):
    gate = np.minimum(gu[..., 0::2], limit)
    return (gu[..., 1::2] + 1.0) * gate / (1.0 + np.exp(-alpha * gate))


def _swiglu_sign(gu, alpha=om.SWIGLU_ALPHA, limit=om.SWIGLU_LIMIT):
    return _real_swiglu(gu, -alpha, limit)


def _mlp_no_b2(xe, W13, b13, W2, b2, alpha=om.SWIGLU_ALPHA, limit=om.SWIGLU_LIMIT):
    return _real_mlp(xe, W13, b13, W2, 0 * b2, alpha, limit)


def _mlp_no_b13(xe, W13, b13, W2, b2, alpha=om.SWIGLU_ALPHA, limit=om.SWIGLU_LIMIT):
    return _real_mlp(xe, W13, 0 * b13, W2, b2, alpha, limit)


def _mlp_transposed_down(xe, W13, b13, W2, b2, alpha=om.SWIGLU_ALPHA, limit=om.SWIGLU_LIMIT):
    h = om.swiglu(xe @ W13.T + b13, alpha, limit)
    return h @ W2 + b2


def _router_no_bias(x_bits, Wr, br):
    return om.bf16_to_f64(x_bits) @ np.asarray(Wr, dtype=np.float64).T


def _topk_ties_high(logits, k):
    T, E = logits.shape
    order = np.argsort(-logits[:, ::-1], axis=1, kind="stable")
    order = E - 1 - order
    ids = order[:, :k]
    srt = np.take_along_axis(logits, order, axis=1)
    gap = srt[:, k - 1] - srt[:, k] if E > k else np.full(T, np.inf)
    return ids, gap


def _softmax_all(logits, ids):
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, ids, axis=1)


def _perm_unstable(ids, E):
    counts, offsets, rows = _real_perm(ids, E)
    rows = rows.copy()
    for e in range(E):
        rows[offsets[e]:offsets[e + 1]] = rows[offsets[e]:offsets[e + 1]][::-1]
    return counts, offsets, rows


def _bad_table():
    t = om.E2M1_TABLE.copy()
    t[5], t[6] = t[6], t[5]
    return t


MUTATIONS = {
    "e2m1_table_entries_swapped": ("E2M1_TABLE", _bad_table),
    "nibbles_swapped": ("dequant_mxfp4", lambda: _dequant_swapped_nibbles),
    "scale_of_wrong_block": ("dequant_mxfp4", lambda: _dequant_wrong_block),
    "scale_bias_126": ("e8m0_scale", lambda: (lambda s: np.ldexp(1.0, np.asarray(s).astype(np.int64) - 126))),
    "gate_up_swapped": ("swiglu", lambda: _swiglu_swapped),
    "no_plus_one": ("swiglu", lambda: _swiglu_no_plus_one),
    "gate_clamped_below": ("swiglu", lambda: _swiglu_two_sided_gate),
    "up_not_clamped": ("swiglu", lambda: _swiglu_no_up_clamp),
    "sigmoid_sign": ("swiglu", lambda: _swiglu_sign),
    "alpha_is_one": ("SWIGLU_ALPHA", lambda: 1.0),
    "limit_is_six": ("SWIGLU_LIMIT", lambda: 6.0),
    "down_bias_dropped": ("expert_mlp", lambda: _mlp_no_b2),
    "gate_up_bias_dropped": ("expert_mlp", lambda: _mlp_no_b13),
    "down_transposed": ("expert_mlp", lambda: _mlp_transposed_down),
    "router_bias_dropped": ("router_logits", lambda: _router_no_bias),
    "ties_to_higher_index": ("select_topk", lambda: _topk_ties_high),
    "softmax_over_all_experts": ("routing_weights", lambda: _softmax_all),
    "permutation_unstable": ("expert_permutation", lambda: _perm_unstable),
}


def _run_all():
    failed = []
    for check in ALL_CHECKS:
        try:
            check()
        except Exception as exc:  # an exception of any kind means the pin caught it
            failed.append((check.__name__, type(exc).__name__))
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, make = MUTATIONS[name]
    value = make()
    monkeypatch.setattr(om, attr, value)
    if attr in ("SWIGLU_ALPHA", "SWIGLU_LIMIT"):
        # defaults were bound at definition time: rebind the users of the constant
        a = value if attr == "SWIGLU_ALPHA" else om.SWIGLU_ALPHA
        l = value if attr == "SWIGLU_LIMIT" else om.SWIGLU_LIMIT
        monkeypatch.setattr(om, "swiglu", lambda gu, alpha=a, limit=l: _real_swiglu(gu, a, l))
    failed = _run_all()
    assert failed, f"mutation {name} passed every pin"
