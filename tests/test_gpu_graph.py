"""The layer captured into a HIP graph and replayed (needs an MI355X).

moe_forward allocates nothing, keeps no state and issues no memsets, so a
whole step (router, permutation, both expert GEMMs, combine) can be captured
once and replayed; this checks that every replay, with eager work of the
same stream in between, reproduces the eager result.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_fp32_amd as moe
from moe_inputs import make_layer_inputs
from tests.gpu_util import to_device, weights_args

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
