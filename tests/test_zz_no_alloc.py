"""moe_forward_noalloc (the layer with the library's own device scratch, for
callers that cannot allocate) against moe_forward, through the C-ABI (needs an
MI355X). Both run the same kernels in the same order, so the outputs must be
equal bit for bit; two calls in a row, the second with fewer tokens, check
that the shared scratch needs no clearing; the first output also meets the
layer's bar against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_fp32_amd as moe
from moe_inputs import make_layer_inputs
from tests.gpu_util import assert_out_close, check_routing, to_device, weights_args

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(0)


# (E, k, first T, second T): the tiled schedule then the weight-streaming one
# (E = 8), and two weight-streaming calls (E = 32, the 20b expert count)
@pytest.mark.parametrize("E,k,T1,T2", [(8, 4, 200, 16), (32, 4, 64, 5)])
def test_forward_noalloc_matches_forward(E, k, T1, T2):
    print(f"forward_noalloc E={E} k={k} T={T1} then T={T2}", flush=True)
    inp = make_layer_inputs(T1, E, k, seed=9100 + E)
    d = to_device(inp)
    outs = []
    for T in (T1, T2):
        x = d["x"][:T]
        out_na = torch.full((T, 2880), float("nan"), dtype=torch.float32, device="cuda")
        moe.forward_noalloc(x, d["Wr"], d["br"], *weights_args(d), out=out_na, k=k)
        out_ref = moe.forward(x, d["Wr"], d["br"], *weights_args(d), k=k)
        torch.cuda.synchronize()
        assert torch.isfinite(out_na).all()
        assert torch.equal(out_na, out_ref), f"T={T}: differs from moe_forward"
        outs.append(out_na)
    ids, w = moe.route(d["x"], d["Wr"], d["br"], k=k)
    ref = oracle.forward(inp, k, ids_override=ids.cpu().numpy())
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["logits"], k)
    assert_out_close(outs[0].cpu().numpy(), ref["out"], "forward_noalloc")


def test_forward_noalloc_refuses_beyond_scratch():
    E, k = 32, 4
    inp = make_layer_inputs(1, E, k, seed=9200)
    d = to_device(inp)
    T = 848   # 3392 routed slots: more than the scratch holds
    assert moe.workspace_size(T, E, k, "forward") > moe._native.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, 2880), dtype=torch.int16, device="cuda")
    out = torch.zeros((T, 2880), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError, match="WORKSPACE"):
        moe.forward_noalloc(x, d["Wr"], d["br"], *weights_args(d), out=out, k=k)
