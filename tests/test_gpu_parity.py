"""HIP path vs the fp64 oracle, through the C-ABI (needs an MI355X).

Routing: top-k sets bit-exact except near-tie tokens; routing weights and
logits to fp32 accuracy. Permutation: bit-exact. Expert outputs and the layer
output: max|err| <= 2e-2 * RMS(ref) and mean per-token relative L2 <= 5e-3.
Small shapes run the whole oracle; the full configurations compare sampled
tokens, and every row of the fused output against the unfused path.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_fp32_amd as moe
from moe_inputs import LAYER_CONFIGS, make_config_inputs, make_layer_inputs
from tests.gpu_util import (assert_out_close, check_routing, expert_edge_tokens, oracle_case,
                            oracle_for_gpu_routing, out_metrics, pack_reference, to_device,
                            weights_args)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(0)


def say(*a):
    print(*a, flush=True)


def np_(t):
    return t.cpu().numpy()


# ---------------------------------------------------------------- library
def test_native_library_is_loaded():
    d = to_device(make_layer_inputs(4, 8, 2, seed=1, router_only=True), pack=False)
    moe.route(d["x"], d["Wr"], d["br"], k=2)
    torch.cuda.synchronize()
    maps = open("/proc/self/maps").read()
    assert moe._native.LIB_PATH in maps


# ---------------------------------------------------------------- packing
@pytest.mark.parametrize("E,N", [(1, 64), (3, 192), (2, 2880), (1, 5760)])
def test_pack_weights_layout(E, N):
    rng = np.random.default_rng(E * 1000 + N)
    codes = rng.integers(0, 256, size=(E, N, 1440), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(E, N, 90), dtype=np.uint8)
    pw = moe.pack_weights(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    assert tuple(pw.codes.shape) == (E, N // 64, 92160)
    assert tuple(pw.scales.shape) == (E, N // 64, 5760)
    want_c, want_s = pack_reference(codes, scales)
    assert np.array_equal(np_(pw.codes).reshape(codes.shape), want_c)
    assert np.array_equal(np_(pw.scales).reshape(scales.shape), want_s)
    # a pure permutation: the byte histograms are unchanged
    assert np.array_equal(np.bincount(np_(pw.codes).ravel(), minlength=256),
                          np.bincount(codes.ravel(), minlength=256))


# ---------------------------------------------------------------- route
# few-token schedule up to T = 128 (T*E <= 4096); above, the register-tiled
# kernel: 12 K splits for E <= 64 (1000, 64), one token tile per wave for
# E = 96 (130, ragged expert tile), 128 (257), 160 (200) and 256 (300), and
# two per wave from 256 blocks of 64 tokens on (16384; 16411 with a ragged
# last block and E = 100)
ROUTE_CASES = [(1, 4, 1), (2, 32, 4), (3, 32, 4), (16, 32, 4), (17, 128, 4), (64, 32, 4),
               (100, 7, 3), (33, 256, 8), (130, 96, 6), (1000, 64, 4), (200, 160, 4),
               (257, 128, 4), (300, 256, 8), (4096, 32, 4), (16384, 128, 4), (16411, 100, 4)]


@pytest.mark.parametrize("T,E,k", ROUTE_CASES)
def test_route(T, E, k):
    say(f"route T={T} E={E} k={k}")
    inp = make_layer_inputs(T, E, k, seed=T * 7 + E, router_only=True)
    d = to_device(inp)
    ids, w, logits = moe.route(d["x"], d["Wr"], d["br"], k=k, return_logits=True)
    torch.cuda.synchronize()
    l64 = oracle.router_logits(inp["x"], inp["Wr"], inp["br"])
    assert np.max(np.abs(np_(logits) - l64)) < 2e-5
    check_routing(np_(ids), np_(w), l64, k)


def test_route_ties_prefer_lower_index():
    inp = make_layer_inputs(8, 16, 4, seed=2, router_only=True)
    inp["Wr"][:] = inp["Wr"][0]
    inp["br"][:] = 0.0
    inp["br"][9] = 0.5
    d = to_device(inp)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=4)
    torch.cuda.synchronize()
    assert np.array_equal(np_(ids), np.tile([9, 0, 1, 2], (8, 1)))
    assert np.allclose(np_(w)[:, 1:], np_(w)[:, 1:2])


def test_route_deterministic():
    inp = make_config_inputs(4, router_only=True)
    d = to_device(inp)
    a = moe.route(d["x"], d["Wr"], d["br"], k=4, return_logits=True)
    b = moe.route(d["x"], d["Wr"], d["br"], k=4, return_logits=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_forward_ragged_two_tile_router():
    """T = 16411 tokens, E = 100: the router's 64-token blocks (a ragged last
    block, a padded expert tile) count the routed slots of each 32-token group,
    and the layer's permutation is built from those counts. Every row of the
    one-call layer against the separate calls (whose permutation counts the
    slots itself), and the first and last routed token of every expert
    against the oracle."""
    T, E, k = 16411, 100, 4
    say(f"forward T={T} E={E} k={k}: router histograms")
    inp = make_layer_inputs(T, E, k, seed=16411)
    d = to_device(inp)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
    out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=k)
    counts, offsets, rows = moe.permute(ids, E)
    y = moe.expert_ffn(d["x"], offsets, rows, *weights_args(d), k=k)
    out_unfused = moe.combine(y, w)
    torch.cuda.synchronize()
    ids_h = np_(ids)
    logits = oracle.router_logits(inp["x"], inp["Wr"], inp["br"])
    check_routing(ids_h, np_(w), logits, k)
    m_all = out_metrics(np_(out), np_(out_unfused).astype(np.float64))
    assert m_all["max_err_over_rms"] < 1e-4, m_all
    sample = np.unique(np.concatenate([[0, T - 1], expert_edge_tokens(ids_h, E)]))
    ref = oracle.forward(inp, k, tokens=sample, ids_override=ids_h)
    m = assert_out_close(np_(out)[sample], ref["out"], "T=16411 E=100")
    say(f"  {sample.size} edge tokens {m}; fused vs unfused {m_all}")


# ---------------------------------------------------------------- permute
def _random_ids(T, E, k, seed, skew=None):
    rng = np.random.default_rng(seed)
    p = None
    if skew is not None:
        p = np.arange(1, E + 1, dtype=np.float64) ** (-skew)
        p /= p.sum()
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=k, replace=False, p=p)
    return ids


PERM_CASES = [(1, 1, 1), (1, 8, 8), (16, 32, 4), (255, 32, 4), (256, 32, 4), (257, 128, 4),
              (1000, 256, 8), (4096, 32, 4), (16384, 128, 4)]


@pytest.mark.parametrize("T,E,k", PERM_CASES)
def test_permute(T, E, k):
    say(f"permute T={T} E={E} k={k}")
    ids = _random_ids(T, E, k, seed=T + E, skew=1.3 if T >= 4096 else None)
    counts, offsets, rows = moe.permute(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    c_ref, o_ref, r_ref = oracle.expert_permutation(ids, E)
    assert np.array_equal(np_(counts), c_ref)
    assert np.array_equal(np_(offsets), o_ref)
    assert np.array_equal(np_(rows), r_ref)


# ---------------------------------------------------------------- experts
# (T, E, k): few rows per expert (T*k <= 28*E at E <= 32, 20*E at E <= 128;
# one 16-token tile per pass up to 10 rows on average, two above) take the
# weight-streaming kernel, more the tiled one
SMALL_CASES = [
    (1, 1, 1),      # one expert: every slot goes to it with weight 1
    (33, 1, 1),     # the same past the schedule threshold (33 > 28 rows): tiled
    (56, 8, 4),     # T*k = 28*E exactly: the last weight-streaming shape (32-token passes)
    (57, 8, 4),     # one token more: the first tiled one
    (1, 4, 4),      # every expert selected
    (5, 8, 2),
    (16, 32, 4),    # the 20b T=16 shape
    (40, 16, 4),    # mean 10 rows: the last shape with 16-token passes
    (44, 16, 4),    # mean 11 rows: the first with 32-token passes
    (30, 8, 4),     # 32-token passes
    (40, 8, 4),     # 32-token passes, experts of more than one pass
    (130, 4, 4),    # tiled: 128-row tile + ragged tail
    (300, 4, 1),    # tiled, k = 1
    (256, 8, 4),
    (192, 64, 4),   # weight-streaming kernels behind the many-token router (T > 128)
    (300, 64, 4),   # the same with two expert tiles in the router
    (600, 64, 4),   # tiled, E = 64
]


def _gpu_route_and_permute(d, E, k):
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
    counts, offsets, rows = moe.permute(ids, E)
    return ids, w, counts, offsets, rows


@pytest.mark.parametrize("T,E,k", SMALL_CASES)
def test_expert_ffn_and_combine(T, E, k):
    say(f"expert_ffn T={T} E={E} k={k}")
    inp = make_layer_inputs(T, E, k, seed=1000 + T + E)
    d = to_device(inp)
    ids, w, counts, offsets, rows = _gpu_route_and_permute(d, E, k)
    y = moe.expert_ffn(d["x"], offsets, rows, *weights_args(d), k=k)
    out = moe.combine(y, w)
    torch.cuda.synchronize()
    ref = oracle.forward(inp, k, ids_override=np_(ids), keep_y=True)
    check_routing(np_(ids), np_(w), ref["logits"], k)
    assert_out_close(np_(y).reshape(T * k, -1), ref["y"].reshape(T * k, -1), "y")
    assert_out_close(np_(out), ref["out"], "combine")


def test_expert_ffn_every_tile_size():
    """Expert row counts on both sides of every 32-token boundary of the tiled
    GEMMs (an expert's last tile loads and multiplies 1, 2, 3 or 4 token
    tiles; 128-row tiles before it), routing fixed by hand (k = 1, E = 16,
    tokens assigned to experts in a shuffled order so the gather is not the
    identity): every slot's y against the oracle."""
    counts = [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 159, 255, 257]
    E, k = len(counts), 1
    T = sum(counts)
    say(f"expert_ffn every tile size: T={T} E={E} counts {counts}")
    inp = make_layer_inputs(T, E, k, seed=6100)
    ids = np.repeat(np.arange(E), counts)[np.random.default_rng(6101).permutation(T)].reshape(T, 1)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = np.argsort(ids[:, 0], kind="stable").astype(np.int32)   # slot t*k + j = t
    d = to_device(inp)
    y = moe.expert_ffn(d["x"], torch.from_numpy(offsets).cuda(), torch.from_numpy(rows).cuda(),
                       *weights_args(d), k=k)
    torch.cuda.synchronize()
    ref = oracle.forward(inp, k, ids_override=ids, keep_y=True)
    m = assert_out_close(np_(y).reshape(T * k, -1), ref["y"].reshape(T * k, -1), "y, every tile size")
    say(f"  metrics {m}")


@pytest.mark.parametrize("T,E,k", SMALL_CASES)
def test_forward_small(T, E, k):
    say(f"forward T={T} E={E} k={k}")
    inp = make_layer_inputs(T, E, k, seed=2000 + T + E)
    d = to_device(inp)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
    out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=k)
    torch.cuda.synchronize()
    ref = oracle.forward(inp, k, ids_override=np_(ids))
    check_routing(np_(ids), np_(w), ref["logits"], k)
    assert_out_close(np_(out), ref["out"], "forward")


def test_forward_max_experts_and_topk():
    """E = 256, k = 8 (the largest supported): few tokens through the
    weight-streaming kernels, and a tiled batch (25 rows per expert) with
    every row against the oracle."""
    for T, E, k in ((6, 256, 8), (800, 256, 8)):
        say(f"forward T={T} E={E} k={k}")
        inp, ref = oracle_case(T, E, k, seed=4000 + T)
        d = to_device(inp)
        ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
        out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=k)
        torch.cuda.synchronize()
        ids_h = np_(ids)
        check_routing(ids_h, np_(w), ref["logits"], k)
        want, _ = oracle_for_gpu_routing(inp, k, ref, ids_h, T)
        m = assert_out_close(np_(out), want, f"E={E} k={k} T={T}")
        say(f"  metrics {m}")


# The 120b expert count (E = 128, k = 4) on one input set of 1024 tokens and
# its prefixes: T*k <= 20*E (T <= 640) takes the weight-streaming kernels
# (grid.y = 128; one 16-token tile per pass up to 10 mean rows, T <= 320,
# two above), T = 641 is the first tiled shape, T = 1024 the tiled kernels
# with 32 mean rows per expert. Every row of every prefix is compared with
# one oracle run over the 1024 tokens.
E128_T = (16, 200, 400, 640, 641, 1024)


@pytest.fixture(scope="module")
def e128():
    inp = make_layer_inputs(max(E128_T), 128, 4, seed=5128)
    say("oracle over 1024 tokens, E=128 (shared by the E=128 cases)")
    ref = oracle.forward(inp, 4, keep_y=True)
    return inp, ref, to_device(inp)


def _prefix(d, T):
    return {key: (v[:T] if key == "x" else v) for key, v in d.items()}


@pytest.mark.parametrize("T", E128_T)
def test_forward_e128(e128, T):
    inp, ref, dfull = e128
    say(f"forward T={T} E=128 k=4 ({'tiled' if T * 4 > 20 * 128 else 'weight-streaming'})")
    d = _prefix(dfull, T)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=4)
    out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=4)
    torch.cuda.synchronize()
    ids_h = np_(ids)
    check_routing(ids_h, np_(w), ref["logits"][:T], 4)
    want, _ = oracle_for_gpu_routing(inp, 4, ref, ids_h, T)
    m = assert_out_close(np_(out), want, f"E=128 T={T}")
    say(f"  metrics {m}")


@pytest.mark.parametrize("T", (200, 641, 1024))
def test_expert_ffn_e128(e128, T):
    """Every routed slot's unweighted expert output (y) against the oracle's."""
    inp, ref, dfull = e128
    say(f"expert_ffn T={T} E=128 k=4")
    d = _prefix(dfull, T)
    ids, w, counts, offsets, rows = _gpu_route_and_permute(d, 128, 4)
    y = moe.expert_ffn(d["x"], offsets, rows, *weights_args(d), k=4)
    out = moe.combine(y, w)
    torch.cuda.synchronize()
    ids_h = np_(ids)
    check_routing(ids_h, np_(w), ref["logits"][:T], 4)
    want_out, want_y = oracle_for_gpu_routing(inp, 4, ref, ids_h, T)
    assert_out_close(np_(y).reshape(T * 4, -1), want_y.reshape(T * 4, -1), "y")
    assert_out_close(np_(out), want_out, "combine")


def test_forward_one_expert_takes_all():
    """A dominant router bias sends every token to one expert (others empty)."""
    for T, E, k, hot in ((40, 8, 2, 5), (400, 4, 1, 2)):
        say(f"forward hot expert T={T} E={E} k={k}")
        inp = make_layer_inputs(T, E, k, seed=31 + T)
        inp["br"][hot] = 50.0
        d = to_device(inp)
        ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
        out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=k)
        torch.cuda.synchronize()
        assert np.all(np_(ids)[:, 0] == hot)
        ref = oracle.forward(inp, k, ids_override=np_(ids))
        assert_out_close(np_(out), ref["out"], "hot expert")


def test_forward_zero_codes_gives_weighted_down_bias():
    T, E, k = 24, 8, 4
    inp = make_layer_inputs(T, E, k, seed=5)
    inp["w13_codes"][:] = 0
    inp["w2_codes"][:] = 0
    d = to_device(inp)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
    out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=k)
    torch.cuda.synchronize()
    b2 = oracle.bf16_to_f64(inp["b2"])
    want = np.einsum("tj,tjh->th", np_(w).astype(np.float64), b2[np_(ids)])
    assert np.max(np.abs(np_(out) - want)) < 1e-6


def test_forward_wide_scale_range():
    """Scale exponents over [-20, +4] instead of [-8, -5]."""
    T, E, k = 48, 8, 4
    inp = make_layer_inputs(T, E, k, seed=6, scale_exp_range=(-20, 4))
    d = to_device(inp)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
    out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=k)
    torch.cuda.synchronize()
    ref = oracle.forward(inp, k, ids_override=np_(ids))
    assert_out_close(np_(out), ref["out"], "scale range")


def test_forward_t0_is_noop():
    inp = make_layer_inputs(1, 8, 2, seed=7)
    d = to_device(inp)
    x0 = d["x"][:0]
    out = moe.forward(x0, d["Wr"], d["br"], *weights_args(d), k=2)
    torch.cuda.synchronize()
    assert out.shape == (0, 2880)


def test_workspace_reuse_and_output_overwrite():
    """A caller-supplied workspace full of garbage and a dirty output buffer."""
    T, E, k = 20, 8, 4
    inp = make_layer_inputs(T, E, k, seed=8)
    d = to_device(inp)
    ws = torch.full((moe.workspace_size(T, E, k),), 0xAB, dtype=torch.uint8, device="cuda")
    out = torch.full((T, 2880), float("nan"), device="cuda")
    a = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=k, out=out, workspace=ws)
    b = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=k, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert torch.allclose(a, b, rtol=1e-5, atol=1e-5)


# ---------------------------------------------------------------- full configs
@pytest.mark.parametrize("idx", [0, 1])
def test_forward_config_full_oracle(idx):
    c = LAYER_CONFIGS[idx]
    say(f"forward config {idx} ({c.name}) against the whole oracle")
    inp = make_config_inputs(idx)
    d = to_device(inp)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=c.k)
    out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=c.k)
    # the same kernels through the separate calls: identical bits (per-slot
    # outputs, then a fixed-order weighted sum)
    counts, offsets, rows = moe.permute(ids, c.E)
    out_calls = moe.combine(moe.expert_ffn(d["x"], offsets, rows, *weights_args(d), k=c.k), w)
    torch.cuda.synchronize()
    assert torch.equal(out, out_calls)
    ref = oracle.forward(inp, c.k, ids_override=np_(ids))
    n_tie = check_routing(np_(ids), np_(w), ref["logits"], c.k)
    m = assert_out_close(np_(out), ref["out"], c.name)
    say(f"  metrics {m} near-tie tokens with another set: {n_tie}")


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_forward_config_sampled(idx):
    """Full configurations: every expert's first and last routed token (its
    first tile and its ragged last tile) plus 62 random tokens against the
    oracle; every row of the one-call layer against the separate calls."""
    c = LAYER_CONFIGS[idx]
    say(f"forward config {idx} ({c.name}): edge + random tokens vs the oracle")
    inp = make_config_inputs(idx)
    d = to_device(inp)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=c.k)
    out = moe.forward(d["x"], d["Wr"], d["br"], *weights_args(d), k=c.k)
    counts, offsets, rows = moe.permute(ids, c.E)
    y = moe.expert_ffn(d["x"], offsets, rows, *weights_args(d), k=c.k)
    out_unfused = moe.combine(y, w)
    torch.cuda.synchronize()
    ids_h = np_(ids)
    logits = oracle.router_logits(inp["x"], inp["Wr"], inp["br"])
    n_tie = check_routing(ids_h, np_(w), logits, c.k)
    # every row: the one-call layer vs the separate calls (expert_ffn + combine)
    m_all = out_metrics(np_(out), np_(out_unfused).astype(np.float64))
    assert m_all["max_err_over_rms"] < 1e-4, m_all
    rng = np.random.default_rng(idx)
    edges = expert_edge_tokens(ids_h, c.E)
    sample = np.unique(np.concatenate([[0, c.T - 1], edges, rng.choice(c.T, 62, replace=False)]))
    touched = np.unique(ids_h[sample])
    assert touched.size == int((np_(counts) > 0).sum()), "every routed expert is sampled"
    ref = oracle.forward(inp, c.k, tokens=sample, ids_override=ids_h, keep_y=True)
    m = assert_out_close(np_(out)[sample], ref["out"], c.name)
    # the sampled rows of the per-slot outputs too (the unfused path's y)
    ref_y = ref["y"]
    yg = np_(y).reshape(c.T, c.k, -1)[sample]
    assert_out_close(yg.reshape(-1, yg.shape[-1]), ref_y.reshape(-1, ref_y.shape[-1]), "y")
    say(f"  {sample.size} tokens ({edges.size} expert edges) metrics {m}; fused vs unfused "
        f"{m_all}; near-tie tokens with another set: {n_tie}")


@pytest.mark.parametrize("T,E,k", [(16, 32, 4), (30, 8, 4), (256, 8, 4)])
def test_gate_up_and_down_accumulate_onto_residual(T, E, k):
    """The two halves as separate calls; the down half adds into a residual."""
    say(f"gate_up + down_accumulate T={T} E={E} k={k}")
    inp = make_layer_inputs(T, E, k, seed=3000 + T + E)
    d = to_device(inp)
    ids, w, counts, offsets, rows = _gpu_route_and_permute(d, E, k)
    h = moe.gate_up(d["x"], offsets, rows, d["experts"], k=k)
    resid = torch.randn((T, 2880), dtype=torch.float32, device="cuda")
    out = resid.clone()
    moe.down_accumulate(h, offsets, rows, w, d["experts"], out=out, k=k)
    torch.cuda.synchronize()
    ref = oracle.forward(inp, k, ids_override=np_(ids))
    assert_out_close(np_(out) - np_(resid).astype(np.float64), ref["out"], "down_accumulate")
