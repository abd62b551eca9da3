"""The MoE sublayer with its neighbours (moe_forward_block, moe_rmsnorm)
against the oracle, through the C-ABI (needs an MI355X).

RMSNorm output: the kernel computes in fp32 and rounds once to bf16, the
oracle rounds the exact value once; they may differ by one bf16 unit where
the fp32 result lands on the other side of a rounding boundary, never more.
The MoE part of the output (out - x) is held to the layer's bar against the
oracle's block on the oracle's own normed input.
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


# Weight-streaming schedule: (1, 4, 1), (16, 32, 4), (100, 40, 4); tiled:
# (128, 8, 8), (130, 2, 2), (256, 8, 4), (300, 4, 1).
BLOCK_CASES = [(1, 4, 1), (16, 32, 4), (100, 40, 4), (128, 8, 8), (130, 2, 2), (256, 8, 4),
               (300, 4, 1)]


@pytest.mark.parametrize("T,E,k", BLOCK_CASES)
def test_forward_block_small(T, E, k):
    say(f"forward_block T={T} E={E} k={k}")
    inp = make_layer_inputs(T, E, k, seed=7000 + T + E)
    g = norm_scale(E)
    d = to_device(inp)
    gd = torch.from_numpy(g).cuda()
    t = moe.rmsnorm(d["x"], gd)
    ids, w = moe.route(t, d["Wr"], d["br"], k=k)
    out = moe.forward_block(d["x"], gd, d["Wr"], d["br"], *weights_args(d), k=k)
    torch.cuda.synchronize()
    t_h = np_(t).view(np.uint16)
    # routing: exact logits of the kernel's own normed input (checked above
    # to within one bf16 unit of the oracle's)
    check_routing(np_(ids), np_(w), oracle.router_logits(t_h, inp["Wr"], inp["br"]), k)
    x64 = oracle.bf16_to_f64(inp["x"])
    # end to end: the oracle's block on its own normed input
    ref = ob.block_forward(inp, k, g, ids_override=np_(ids))
    m = assert_out_close(np_(out) - x64, ref["out"] - x64, "forward_block")
    say(f"  metrics (out - x) {m}")


@pytest.mark.parametrize("idx", [1, 4])
def test_forward_block_config(idx):
    c = LAYER_CONFIGS[idx]
    say(f"forward_block config {idx} ({c.name})")
    inp = make_config_inputs(idx)
    g = norm_scale(idx)
    d = to_device(inp)
    gd = torch.from_numpy(g).cuda()
    t = moe.rmsnorm(d["x"], gd)
    ids, w = moe.route(t, d["Wr"], d["br"], k=c.k)
    out = moe.forward_block(d["x"], gd, d["Wr"], d["br"], *weights_args(d), k=c.k)
    # the block equals the layer on the normed input plus the residual, row for row
    out_layer = moe.forward(t, d["Wr"], d["br"], *weights_args(d), k=c.k)
    torch.cuda.synchronize()
    x64 = oracle.bf16_to_f64(inp["x"])
    assert np.max(np.abs((np_(out) - x64) - np_(out_layer))) <= 1e-4 * np.sqrt(np.mean(np_(out_layer) ** 2))
    sample = None if c.T <= 64 else np.unique(np.concatenate(
        [[0, c.T - 1], np.random.default_rng(idx).choice(c.T, 30, replace=False)]))
    n_tie = check_routing(np_(ids), np_(w),
                          oracle.router_logits(np_(t).view(np.uint16), inp["Wr"], inp["br"]), c.k)
    ref = ob.block_forward(inp, c.k, g, tokens=sample, ids_override=np_(ids))
    got = np_(out) if sample is None else np_(out)[sample]
    xs = x64 if sample is None else x64[sample]
    m = assert_out_close(got - xs, ref["out"] - xs, c.name)
    say(f"  metrics (out - x) {m}; near-tie tokens with another set: {n_tie}")
