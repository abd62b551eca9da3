"""The layer captured into a HIP graph and replayed (needs an MI355X).

moe_forward allocates nothing, keeps no state and issues no memsets, so a
whole step (router, permutation, both expert GEMMs, combine) can be captured
once and replayed; this checks that every replay, with eager work of the
same stream in between, reproduces the eager result bit for bit, and that
the replayed output meets the layer's bar against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.block as ob
import sparse_moe_ffn_fp32_amd as moe
from moe_inputs import make_layer_inputs
from tests.gpu_util import assert_out_close, check_routing, to_device, weights_args

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(0)


# (T, E, k, path): the weight-streaming schedule (T=64, E=32; T=16 with the
# norm and residual) and the tiled one, bf16 and FP6 pieces. Both schedules
# sum a token's k expert outputs in a fixed order, so every replay must
# reproduce the eager output bit for bit.
@pytest.mark.parametrize("T,E,k,path", [(64, 32, 4, "bf16"), (256, 8, 4, "bf16"),
                                        (256, 8, 4, "mx6"), (16, 32, 4, "block")])
def test_forward_graph_replays(T, E, k, path):
    print(f"graph T={T} E={E} k={k} {path}", flush=True)
    inp = make_layer_inputs(T, E, k, seed=9000 + T + E)
    d = to_device(inp)
    args = weights_args(d)
    ws = torch.empty(moe.workspace_size(T, E, k), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, 2880), dtype=torch.float32, device="cuda")
    g = torch.ones(2880, dtype=torch.float32, device="cuda") * 1.5

    def step():
        if path == "block":
            moe.forward_block(d["x"], g, d["Wr"], d["br"], *args, k=k, out=out, workspace=ws)
        elif path == "mx6":
            moe.forward_mx6(d["x"], d["Wr"], d["br"], *args, k=k, out=out, workspace=ws)
        else:
            moe.forward(d["x"], d["Wr"], d["br"], *args, k=k, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        out.fill_(float("nan"))            # eager work between replays
        ws.fill_(0xCD)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        assert torch.isfinite(got).all(), f"replay {r}: non-finite"
        assert torch.equal(got, eager), f"replay {r} differs"
    # the replayed output against the oracle (the block: the routing the
    # replay left in the workspace against the oracle's routing of the normed
    # input, and out - x against the oracle's block)
    torch.cuda.synchronize()
    if path == "block":
        ids, w = moe.workspace_routing(ws, T, k)
        g64 = np.full(2880, 1.5, dtype=np.float32)
        check_routing(ids.cpu().numpy(), w.cpu().numpy(),
                      oracle.router_logits_f64(ob.rmsnorm(inp["x"], g64), inp["Wr"], inp["br"]), k)
        ref = ob.block_forward(inp, k, g64, ids_override=ids.cpu().numpy())
        x64 = oracle.bf16_to_f64(inp["x"])
        assert_out_close(got.cpu().numpy() - x64, ref["out"] - x64, "graph replay, block")
    else:
        ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
        ref = oracle.forward(inp, k, ids_override=ids.cpu().numpy())
        check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["logits"], k)
        assert_out_close(got.cpu().numpy(), ref["out"], f"graph replay, {path}")


def test_forward_graph_pass_of_layers():
    """Three layer steps with different weights (a decode pass through three
    MoE layers, T=64, E=32) captured in one graph, one workspace shared: every
    replay reproduces each layer's eager output bit for bit, and the first
    layer's output meets the bar against the oracle."""
    T, E, k = 64, 32, 4
    print(f"graph pass: 3 layers T={T} E={E} k={k}", flush=True)
    inps = [make_layer_inputs(T, E, k, seed=9100 + j) for j in range(3)]
    ds = [to_device(inp) for inp in inps]
    x = ds[0]["x"]
    ws = torch.empty(moe.workspace_size(T, E, k), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((T, 2880), dtype=torch.float32, device="cuda") for _ in range(3)]

    def layers():
        for d, out in zip(ds, outs):
            moe.forward(x, d["Wr"], d["br"], *weights_args(d), k=k, out=out, workspace=ws)

    layers()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layers()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layers()
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        ws.fill_(0xCD)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"replay {r}, layer {j} differs"
    ids, w = moe.route(x, ds[0]["Wr"], ds[0]["br"], k=k)
    ref = oracle.forward(dict(inps[0], x=inps[0]["x"]), k, ids_override=ids.cpu().numpy())
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["logits"], k)
    assert_out_close(outs[0].cpu().numpy(), ref["out"], "graph pass, layer 0")
