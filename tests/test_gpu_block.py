"""The MoE sublayer with its neighbours (moe_forward_block, moe_rmsnorm)
against the oracle, through the C-ABI (needs an MI355X).

RMSNorm output: the kernel computes in fp32 and rounds once to bf16, the
oracle rounds the exact value once; they may differ by one bf16 unit where
the fp32 result lands on the other side of a rounding boundary, never more.
Routing: the expert sets the block call leaves in its workspace against the
oracle's routing of the unrounded normed input (bit-exact outside near
ties). The MoE part of the output (out - x) is held to the layer's bar
against the oracle's block.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.block as ob
import sparse_moe_ffn_fp32_amd as moe
from moe_inputs import LAYER_CONFIGS, bf16_bits_from_f32, make_config_inputs, make_layer_inputs
from tests.gpu_util import assert_out_close, check_routing, to_device, weights_args

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


def norm_scale(seed):
    return np.random.default_rng(seed).uniform(0.5, 2.0, 2880).astype(np.float32)


def assert_bf16_within_one_unit(got_bits, want_bits):
    g = got_bits.astype(np.int32)
    w = want_bits.astype(np.int32)
    # same sign and magnitude codes one apart at most (bf16 bit patterns of
    # same-sign values are ordered like the values)
    same_sign = (g >> 15) == (w >> 15)
    diff = np.abs(g - w)
    ok = (diff == 0) | (same_sign & (diff <= 1))
    assert ok.all(), (np.argwhere(~ok)[:5], g[~ok][:5], w[~ok][:5])
    return float((diff != 0).mean())


@pytest.mark.parametrize("T,eps", [(1, 1e-5), (37, 1e-5), (1024, 1e-5), (64, 0.5)])
def test_rmsnorm(T, eps):
    rng = np.random.default_rng(T)
    x = (rng.standard_normal((T, 2880)) * np.exp(rng.uniform(-4, 4, (T, 1)))).astype(np.float32)
    x[0, :7] = 0.0
    xb = bf16_bits_from_f32(x)
    g = norm_scale(T)
    t = moe.rmsnorm(torch.from_numpy(xb.view(np.int16)).cuda(), torch.from_numpy(g).cuda(), eps)
    torch.cuda.synchronize()
    frac = assert_bf16_within_one_unit(np_(t).view(np.uint16), ob.normed_input_bits(xb, g, eps))
    say(f"rmsnorm T={T} eps={eps}: {frac:.2e} of values one bf16 unit apart")
    assert frac < 1e-2


def block_call(d, gd, T, E, k):
    """forward_block on its own workspace; returns out and the routing it left."""
    ws = torch.empty(moe.workspace_size(T, E, k, "forward_block"), dtype=torch.uint8, device="cuda")
    out = moe.forward_block(d["x"], gd, d["Wr"], d["br"], *weights_args(d), k=k, workspace=ws)
    ids, w = moe.workspace_routing(ws, T, k)
    torch.cuda.synchronize()
    return np_(out), np_(ids), np_(w)


def router_logits_of_block(inp, g):
    """The oracle's router logits of the block: on the unrounded normed input."""
    return oracle.router_logits_f64(ob.rmsnorm(inp["x"], g), inp["Wr"], inp["br"])


# Norm folded into the router and the weight-streaming gate/up (T <= 128,
# T*E <= 4096): (1, 4, 1), (16, 32, 4), (100, 40, 4), (128, 32, 4) (the
# largest: T*E = 4096), (8, 256, 4) (eight expert tiles per router wave, one
# token per finish block); the norm kernel with the
# weight-streaming GEMMs on its output (many-token router, K-split and
# expert-tiled): (200, 32, 4), (160, 80, 4); with the tiled GEMMs: (128, 8, 8)
# (few-token router), (130, 2, 2), (256, 8, 4), (300, 4, 1).
BLOCK_CASES = [(1, 4, 1), (16, 32, 4), (100, 40, 4), (128, 32, 4), (8, 256, 4), (200, 32, 4), (160, 80, 4), (128, 8, 8),
               (130, 2, 2), (256, 8, 4), (300, 4, 1)]


@pytest.mark.parametrize("T,E,k", BLOCK_CASES)
def test_forward_block_small(T, E, k):
    say(f"forward_block T={T} E={E} k={k}")
    inp = make_layer_inputs(T, E, k, seed=7000 + T + E)
    g = norm_scale(E)
    d = to_device(inp)
    gd = torch.from_numpy(g).cuda()
    out, ids, w = block_call(d, gd, T, E, k)
    n_tie = check_routing(ids, w, router_logits_of_block(inp, g), k)
    x64 = oracle.bf16_to_f64(inp["x"])
    # at most 24 tokens through the oracle's experts where many experts are touched
    sample = None if T * E <= 8192 else np.unique(np.concatenate(
        [[0, T - 1], np.random.default_rng(T).choice(T, 22, replace=False)]))
    ref = ob.block_forward(inp, k, g, tokens=sample, ids_override=ids)
    got = out if sample is None else out[sample]
    xs = x64 if sample is None else x64[sample]
    m = assert_out_close(got - xs, ref["out"] - xs, "forward_block")
    say(f"  metrics (out - x) {m}; near-tie tokens with another set: {n_tie}")


@pytest.mark.parametrize("idx", [1, 4])
def test_forward_block_config(idx):
    c = LAYER_CONFIGS[idx]
    say(f"forward_block config {idx} ({c.name})")
    inp = make_config_inputs(idx)
    g = norm_scale(idx)
    d = to_device(inp)
    gd = torch.from_numpy(g).cuda()
    out, ids, w = block_call(d, gd, c.T, c.E, c.k)
    x64 = oracle.bf16_to_f64(inp["x"])
    sample = None if c.T <= 64 else np.unique(np.concatenate(
        [[0, c.T - 1], np.random.default_rng(idx).choice(c.T, 30, replace=False)]))
    n_tie = check_routing(ids, w, router_logits_of_block(inp, g), c.k)
    ref = ob.block_forward(inp, c.k, g, tokens=sample, ids_override=ids)
    got = out if sample is None else out[sample]
    xs = x64 if sample is None else x64[sample]
    m = assert_out_close(got - xs, ref["out"] - xs, c.name)
    say(f"  metrics (out - x) {m}; near-tie tokens with another set: {n_tie}")
