"""Pins of the fp64 oracle against things other than itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with what the
pages or the mathematics fix. They are collected by ``test_oracle.py`` and
re-run by ``test_oracle_mutations.py`` against deliberately broken copies of
the oracle, to show that a plausible mistake anywhere in it is caught.

Independent routes used here (none of them calls the oracle's own helpers):
bit-field decoding of E2M1 / E8M0 / bf16 written from the format definitions,
pure-Python loops for tiny layers, closed forms for structured weights, and a
dense all-experts mixture written with numpy.einsum.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

import oracle.moe_oracle as om
from moe_inputs import make_layer_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gpt_oss_page_figures.json")


# ---------------------------------------------------------------- bit formulas
def e2m1_from_bits(c: int) -> float:
    """FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    sign = -1.0 if c & 0x8 else 1.0
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = m * 0.5 if e == 0 else (2.0 ** (e - 1)) * (1.0 + 0.5 * m)
    return sign * mag


def e8m0_from_bits(s: int) -> float:
    """E8M0 byte s -> 2^(s-127), built as the float64 with that exponent field."""
    return struct.unpack("<d", struct.pack("<Q", (s - 127 + 1023) << 52))[0]


def bf16_from_bits(b: int) -> float:
    sign = -1.0 if b & 0x8000 else 1.0
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0:
        return sign * (m / 128.0) * 2.0 ** -126
    return sign * (1.0 + m / 128.0) * 2.0 ** (e - 127)


def dequant_by_bits(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Python-loop dequantisation of one [N, K/2] matrix from the bit formulas."""
    N, Kh = codes.shape
    W = np.zeros((N, 2 * Kh))
    for n in range(N):
        for b in range(Kh):
            byte = int(codes[n, b])
            sc = e8m0_from_bits(int(scales[n, (2 * b) // 32]))
            W[n, 2 * b] = e2m1_from_bits(byte & 0xF) * sc
            W[n, 2 * b + 1] = e2m1_from_bits(byte >> 4) * sc
    return W


# ---------------------------------------------------------------- pure-Python layer
def brute_force_layer(inp, k, alpha=1.702, limit=7.0):
    """Every expert on every token with Python loops; dense mixture with the
    full softmax masked to the top-k set and renormalised."""
    x = [[bf16_from_bits(int(v)) for v in row] for row in inp["x"]]
    T, H = len(x), len(x[0])
    E = inp["Wr"].shape[0]
    I2 = inp["w13_codes"].shape[1]
    W13 = [dequant_by_bits(inp["w13_codes"][e], inp["w13_scales"][e]) for e in range(E)]
    W2 = [dequant_by_bits(inp["w2_codes"][e], inp["w2_scales"][e]) for e in range(E)]
    b13 = [[bf16_from_bits(int(v)) for v in inp["b13"][e]] for e in range(E)]
    b2 = [[bf16_from_bits(int(v)) for v in inp["b2"][e]] for e in range(E)]
    out = np.zeros((T, H))
    ids_all = []
    for t in range(T):
        logit = [sum(x[t][h] * float(inp["Wr"][e, h]) for h in range(H)) + float(inp["br"][e])
                 for e in range(E)]
        chosen = sorted(range(E), key=lambda e: (-logit[e], e))[:k]
        ids_all.append(chosen)
        mx = max(logit)
        p = [math.exp(l - mx) for l in logit]
        z = sum(p[e] for e in chosen)
        for e in range(E):
            gu = [sum(W13[e][n, h] * x[t][h] for h in range(H)) + b13[e][n] for n in range(I2)]
            hvec = []
            for i in range(I2 // 2):
                g = min(gu[2 * i], limit)
                u = max(min(gu[2 * i + 1], limit), -limit)
                hvec.append((u + 1.0) * g / (1.0 + math.exp(-alpha * g)))
            y = [sum(W2[e][n, i] * hvec[i] for i in range(I2 // 2)) + b2[e][n] for n in range(H)]
            wt = p[e] / z if e in chosen else 0.0
            for n in range(H):
                out[t, n] += wt * y[n]
    return out, np.array(ids_all)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- pins
def check_e2m1_table():
    for c in range(16):
        want = e2m1_from_bits(c)
        got = float(om.E2M1_TABLE[c])
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (c, got, want)
    # the table through the dequantiser, for every byte (both nibbles)
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    scales = np.full((8, 2), 127, dtype=np.uint8)
    W = om.dequant_mxfp4(codes, scales)
    for byte in range(256):
        n, b = divmod(byte, 32)
        assert W[n, 2 * b] == e2m1_from_bits(byte & 0xF), byte
        assert W[n, 2 * b + 1] == e2m1_from_bits(byte >> 4), byte


def check_e8m0_scales():
    s = np.arange(255)
    got = om.e8m0_scale(s)
    for v in range(255):
        assert got[v] == e8m0_from_bits(v), v
    assert np.isnan(om.e8m0_scale(np.array([255]))[0])


def check_bf16_decode():
    rng = np.random.default_rng(11)
    bits = np.concatenate([rng.integers(0, 65536, 4000), [0, 0x8000, 0x0001, 0x807F, 0x3F80, 0xC0E0]])
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)  # finite only
    got = om.bf16_to_f64(bits)
    want = np.array([bf16_from_bits(int(b)) for b in bits])
    assert np.array_equal(got, want)


def check_dequant_positions():
    """One non-zero code at an odd K in block 1: pins nibble order and scale index."""
    codes = np.zeros((3, 32), dtype=np.uint8)   # K = 64, two blocks
    scales = np.full((3, 2), 127, dtype=np.uint8)
    codes[1, 17] = 0xA3                          # K = 34 (low) and 35 (high)
    scales[1, 1] = 130                           # block 1 -> x8
    scales[1, 0] = 120                           # must not be used for K = 34, 35
    W = om.dequant_mxfp4(codes, scales)
    want = np.zeros((3, 64))
    want[1, 34] = 1.5 * 8.0
    want[1, 35] = -1.0 * 8.0
    assert np.array_equal(W, want)


def check_routing_weights():
    inp = make_layer_inputs(T=24, E=9, k=3, seed=3, H=64, I=32)
    logits, ids, w, gap = om.route(inp, 3)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-14)
    sel = np.take_along_axis(logits, ids, axis=1)
    for a in range(3):
        for b in range(3):
            assert np.allclose(w[:, a] / w[:, b], np.exp(sel[:, a] - sel[:, b]), rtol=1e-12)
    # descending logits, and the k-th beats every unselected expert
    assert np.all(np.diff(sel, axis=1) <= 0)
    for t in range(24):
        rest = np.setdiff1d(np.arange(9), ids[t])
        assert np.all(logits[t, rest] <= sel[t, -1])
        assert np.isclose(gap[t], sel[t, -1] - logits[t, rest].max())


def check_topk_ties():
    """Identical router rows and biases force ties: lower expert index first."""
    inp = make_layer_inputs(T=5, E=6, k=3, seed=4, H=32, I=32)
    inp["Wr"][:] = inp["Wr"][0]
    inp["br"][:] = 0.0
    _, ids, w, gap = om.route(inp, 3)
    assert np.array_equal(ids, np.tile([0, 1, 2], (5, 1)))
    assert np.allclose(w, 1.0 / 3.0) and np.all(gap == 0)
    # a strict winner at a high index goes first
    inp["br"][4] = 1.0
    _, ids, _, _ = om.route(inp, 3)
    assert np.array_equal(ids, np.tile([4, 0, 1], (5, 1)))


def check_permutation_invariants():
    rng = np.random.default_rng(5)
    T, E, k = 37, 7, 3
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    counts, offsets, rows = om.expert_permutation(ids, E)
    flat = ids.reshape(-1)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.sort(rows), np.arange(T * k))
    for e in range(E):
        seg = rows[offsets[e]:offsets[e + 1]]
        assert seg.size == counts[e] == np.count_nonzero(flat == e)
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def check_brute_force_tiny():
    for (T, E, k, seed) in [(3, 5, 2, 21), (2, 4, 4, 22), (1, 1, 1, 23)]:
        inp = make_layer_inputs(T=T, E=E, k=k, seed=seed, H=64, I=32)
        want, ids = brute_force_layer(inp, k)
        res = om.forward(inp, k)
        assert np.array_equal(res["ids"], ids), (res["ids"], ids)
        assert _rel(res["out"], want) < 1e-12, _rel(res["out"], want)


def check_zero_codes():
    """All-zero codes: every expert output is its down bias b2."""
    inp = make_layer_inputs(T=11, E=6, k=2, seed=6, H=64, I=32)
    inp["w13_codes"][:] = 0
    inp["w2_codes"][:] = 0
    res = om.forward(inp, 2)
    b2 = np.array([[bf16_from_bits(int(v)) for v in row] for row in inp["b2"]])
    want = np.zeros((11, 64))
    for t in range(11):
        for j in range(2):
            want[t] += res["w"][t, j] * b2[res["ids"][t, j]]
    assert _rel(res["out"], want) < 1e-14


def _single_code_layer(x_vals, g_code, u_code, g_scale, u_scale, seed=8):
    """E = k = 1, H = I = 32 (one MX block). Gate row 2i reads K = i, up row
    2i+1 reads K = (i+1) % 32, down row n reads K = (3n+1) % 32 with value 1."""
    H = I = 32
    inp = make_layer_inputs(T=len(x_vals), E=1, k=1, seed=seed, H=H, I=I)
    from moe_inputs import bf16_bits_from_f32
    inp["x"] = bf16_bits_from_f32(np.array(x_vals, dtype=np.float32))
    c13 = np.zeros((1, 2 * I, H // 2), dtype=np.uint8)
    s13 = np.zeros((1, 2 * I, 1), dtype=np.uint8)
    for i in range(I):
        for row, kk, code, sc in ((2 * i, i, g_code, g_scale), (2 * i + 1, (i + 1) % H, u_code, u_scale)):
            c13[0, row, kk // 2] |= code << (4 * (kk % 2))
            s13[0, row, 0] = sc
    c2 = np.zeros((1, H, I // 2), dtype=np.uint8)
    s2 = np.full((1, H, 1), 127, dtype=np.uint8)
    for n in range(H):
        kk = (3 * n + 1) % I
        c2[0, n, kk // 2] |= 0x2 << (4 * (kk % 2))           # code 2 -> 1.0
    inp.update(w13_codes=c13, w13_scales=s13, w2_codes=c2, w2_scales=s2)
    return inp


def check_single_code_closed_form():
    rng = np.random.default_rng(9)
    xs = [list(rng.standard_normal(32) * 3.0) for _ in range(3)]
    xs.append([6.0] * 16 + [-6.0] * 16)     # drives gate above 7 and up beyond +-7
    for g_code, u_code, g_sc, u_sc in ((0x7, 0x6, 128, 128), (0x5, 0xD, 127, 128), (0xB, 0x3, 126, 129)):
        inp = _single_code_layer(xs, g_code, u_code, g_sc, u_sc)
        res = om.forward(inp, 1)
        b13 = [bf16_from_bits(int(v)) for v in inp["b13"][0]]
        b2 = [bf16_from_bits(int(v)) for v in inp["b2"][0]]
        gv = e2m1_from_bits(g_code) * 2.0 ** (g_sc - 127)
        uv = e2m1_from_bits(u_code) * 2.0 ** (u_sc - 127)
        clamped = 0
        for t in range(len(xs)):
            xt = [bf16_from_bits(int(v)) for v in inp["x"][t]]
            h = []
            for i in range(32):
                g = xt[i] * gv + b13[2 * i]
                u = xt[(i + 1) % 32] * uv + b13[2 * i + 1]
                clamped += (g > 7) + (abs(u) > 7)
                g = min(g, 7.0)
                u = max(-7.0, min(u, 7.0))
                h.append((u + 1.0) * g / (1.0 + math.exp(-1.702 * g)))
            want = [h[(3 * n + 1) % 32] + b2[n] for n in range(32)]
            assert np.allclose(res["out"][t], want, rtol=1e-13, atol=1e-13), (t, res["out"][t], want)
        assert clamped > 0


def check_swiglu_clamp_values():
    gu = np.array([[10.0, 10.0, 10.0, -10.0, -3.0, 0.5, 7.0, -7.0]])
    got = om.swiglu(gu)
    s = lambda g: 1.0 / (1.0 + math.exp(-1.702 * g))
    want = [(7 + 1) * 7 * s(7), (-7 + 1) * 7 * s(7), (0.5 + 1) * -3 * s(-3), (-7 + 1) * 7 * s(7)]
    assert np.allclose(got[0], want, rtol=1e-14)


def check_equivariance():
    inp = make_layer_inputs(T=9, E=6, k=2, seed=12, H=64, I=32)
    base = om.forward(inp, 2)
    perm = np.random.default_rng(1).permutation(9)
    inp_p = dict(inp, x=inp["x"][perm])
    res = om.forward(inp_p, 2)
    assert _rel(res["out"], base["out"][perm]) < 1e-13
    # relabel the experts: router rows, biases and weight sets move together
    q = np.random.default_rng(2).permutation(6)
    inp_q = dict(inp)
    for key in ("Wr", "br", "w13_codes", "w13_scales", "b13", "w2_codes", "w2_scales", "b2"):
        inp_q[key] = inp[key][q]
    res = om.forward(inp_q, 2)
    assert _rel(res["out"], base["out"]) < 1e-13
    assert np.array_equal(q[res["ids"]], base["ids"])


def check_dense_mixture_reduction():
    """Scale bytes 127 and k = E: a softmax-weighted sum of dense SwiGLU MLPs."""
    T, E, H, I = 6, 3, 64, 32
    inp = make_layer_inputs(T=T, E=E, k=E, seed=13, H=H, I=I)
    inp["w13_scales"][:] = 127
    inp["w2_scales"][:] = 127
    res = om.forward(inp, E)
    lut = np.array([e2m1_from_bits(c) for c in range(16)])
    def dense(codes):
        W = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,))
        W[..., 0::2] = lut[codes & 15]
        W[..., 1::2] = lut[codes >> 4]
        return W
    W13, W2 = dense(inp["w13_codes"]), dense(inp["w2_codes"])
    tobf = np.vectorize(lambda b: bf16_from_bits(int(b)))
    x = tobf(inp["x"])
    b13, b2 = tobf(inp["b13"]), tobf(inp["b2"])
    logits = np.einsum("th,eh->te", x, inp["Wr"].astype(np.float64)) + inp["br"]
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    gu = np.einsum("th,enh->ten", x, W13) + b13[None]
    g = np.minimum(gu[..., 0::2], 7.0)
    u = np.clip(gu[..., 1::2], -7.0, 7.0)
    h = (u + 1) * g / (1 + np.exp(-1.702 * g))
    y = np.einsum("tei,eni->ten", h, W2) + b2[None]
    want = np.einsum("te,ten->tn", p, y)
    assert _rel(res["out"], want) < 1e-12


def check_parameter_count():
    """The expert and router shapes reproduce the 20b checkpoint total exactly."""
    with open(GOLDEN) as f:
        g = json.load(f)
    cf = g["config_fields"]
    H, I = cf["hidden_size"], cf["intermediate_size"]
    nq, nkv, hd, V = cf["num_attention_heads"], cf["num_key_value_heads"], cf["head_dim"], cf["vocab_size"]
    size = lambda shp: int(np.prod(shp))
    expert = sum(size(s) for s in om.expert_parameter_shapes(H, I).values())
    # attention with q/k/v/o biases and one learned sink per head (the
    # techniques map's "Learnable attention sink" row), two RMSNorms per layer
    attn = (nq * hd * H + nq * hd) + 2 * (nkv * hd * H + nkv * hd) + (H * nq * hd + H) + nq
    def total(E, L, active=False):
        router = sum(size(s) for s in om.router_parameter_shapes(H, E).values())
        n_exp = cf["experts_per_token"] if active else E
        layer = attn + 2 * H + router + n_exp * expert
        emb = (V * H) * (1 if active else 2)
        return L * layer + emb + H
    t20 = total(cf["num_local_experts_20b"], cf["num_hidden_layers_20b"])
    assert t20 == g["checkpoint_parameters_20b"]["value"], t20
    t120 = total(cf["num_local_experts_120b"], cf["num_hidden_layers_120b"])
    assert round(t120 / 1e9, 1) == g["total_parameters_120b_billions"]["value"], t120
    # active per token: k experts, LM head counted, embedding lookup not
    a20 = total(cf["num_local_experts_20b"], cf["num_hidden_layers_20b"], active=True)
    a120 = total(cf["num_local_experts_120b"], cf["num_hidden_layers_120b"], active=True)
    assert round(a20 / 1e9, 1) == g["active_parameters_20b_billions"]["value"], a20
    assert round(a120 / 1e9, 1) == g["active_parameters_120b_billions"]["value"], a120


def check_restricted_tokens_and_override():
    """Computing a subset of tokens, or forcing the expert sets, agrees with the full run."""
    inp = make_layer_inputs(T=10, E=5, k=2, seed=14, H=64, I=32)
    full = om.forward(inp, 2, keep_y=True)
    sub = om.forward(inp, 2, tokens=[7, 2, 9])
    assert _rel(sub["out"], full["out"][[7, 2, 9]]) < 1e-14
    forced = om.forward(inp, 2, ids_override=full["ids"][:, ::-1])
    assert _rel(forced["out"], full["out"]) < 1e-13
    # y rows recombine to out
    recomb = np.einsum("tj,tjh->th", full["w"], full["y"])
    assert _rel(recomb, full["out"]) < 1e-13


ALL_CHECKS = [
    check_e2m1_table, check_e8m0_scales, check_bf16_decode, check_dequant_positions,
    check_routing_weights, check_topk_ties, check_permutation_invariants,
    check_brute_force_tiny, check_zero_codes, check_single_code_closed_form,
    check_swiglu_clamp_values, check_equivariance, check_dense_mixture_reduction,
    check_parameter_count, check_restricted_tokens_and_override,
]
