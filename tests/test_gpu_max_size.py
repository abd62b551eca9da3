"""The layer at the largest routed-slot count the C-ABI accepts
(T*k = MOE_MAX_ROUTED = 4,194,304: T = 1,048,576 tokens, k = 4, E = 32),
through the C-ABI (needs an MI355X; about 120 GB of device memory).

At this size the oracle cannot run the whole layer, so the test checks what
is unique at any size and samples what is not:
  * the expert permutation of all 4,194,304 slots, bit for bit against the
    oracle's stable counting sort of the GPU's own routing ids;
  * first, last and random tokens: routing against the float64 logits, and
    the output of both tiled paths (bf16 and block-scaled FP4 x FP6) against
    the oracle, to the layer's bar;
  * every row: the FP6-piece path against the bf16 path, to the same bar.
The activations are drawn on the device (same distribution as the host
draw); the sampled rows are read back for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_fp32_amd as moe
from moe_inputs import device_activations, make_layer_inputs
from tests.gpu_util import MAX_ERR_OVER_RMS, MEAN_REL_L2, assert_out_close, check_routing, to_device, weights_args

pytestmark = pytest.mark.gpu

MAX_ROUTED = 4194304   # MOE_MAX_ROUTED in include/moe.h


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(0)


def say(*a):
    print(*a, flush=True)


def np_(t):
    return t.cpu().numpy()


def rows_close_on_device(got, ref, chunk=1 << 15):
    """max |got - ref| / RMS(ref) and mean per-token relative L2, in float64
    on the device, chunk by chunk."""
    sq = 0.0
    max_abs = 0.0
    rel_sum = 0.0
    T = ref.shape[0]
    for r0 in range(0, T, chunk):
        g = got[r0:r0 + chunk].double()
        f = ref[r0:r0 + chunk].double()
        err = g - f
        sq += float((f * f).sum())
        max_abs = max(max_abs, float(err.abs().max()))
        nt = f.norm(dim=1)
        rel_sum += float((err.norm(dim=1) / torch.where(nt > 0, nt, torch.ones_like(nt))).sum())
    rms = (sq / (T * ref.shape[1])) ** 0.5
    return dict(max_err_over_rms=max_abs / rms, mean_rel_l2=rel_sum / T)


def test_forward_max_routed_slots():
    E, k = 32, 4
    T = MAX_ROUTED // k
    assert moe.workspace_size(T, E, k) > 0
    with pytest.raises(ValueError):
        moe.workspace_size(T + 1, E, k)     # one token past the limit is refused
    say(f"max size: T={T} E={E} k={k} (T*k={T * k})")
    inp = make_layer_inputs(1, E, k, seed=4242)     # router and expert parameters
    d = to_device(inp)
    x = device_activations(T, seed=4242)
    ids, w = moe.route(x, d["Wr"], d["br"], k=k)
    counts, offsets, rows = moe.permute(ids, E)
    torch.cuda.synchronize()
    say("  routed and permuted")
    ids_h = np_(ids)
    c_ref, o_ref, r_ref = oracle.expert_permutation(ids_h, E)
    assert np.array_equal(np_(counts), c_ref)
    assert np.array_equal(np_(offsets), o_ref)
    assert np.array_equal(np_(rows), r_ref)
    say(f"  permutation of {T * k} slots exact; rows per expert {int(c_ref.min())}..{int(c_ref.max())}")
    del counts, offsets, rows

    out = moe.forward(x, d["Wr"], d["br"], *weights_args(d), k=k)
    torch.cuda.synchronize()
    say("  forward (bf16) done")
    out6 = moe.forward_mx6(x, d["Wr"], d["br"], *weights_args(d), k=k)
    torch.cuda.synchronize()
    say("  forward_mx6 done")

    rng = np.random.default_rng(4242)
    sample = np.unique(np.concatenate([[0, 1, T // 2, T - 2, T - 1], rng.choice(T, 27, replace=False)]))
    xs = np_(x[torch.from_numpy(sample).cuda()]).view(np.uint16)
    ref = oracle.forward(dict(inp, x=xs), k, ids_override=ids_h[sample])
    n_tie = check_routing(ids_h[sample], np_(w)[sample], ref["logits"], k)
    sel = torch.from_numpy(sample).cuda()
    m = assert_out_close(np_(out[sel]), ref["out"], "forward at max size")
    m6 = assert_out_close(np_(out6[sel]), ref["out"], "forward_mx6 at max size")
    say(f"  sampled: bf16 {m}; mx6 {m6}; near-tie tokens with another set: {n_tie}")

    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(out6).all())
    mall = rows_close_on_device(out6, out)
    say(f"  every row, mx6 vs bf16: {mall}")
    assert mall["max_err_over_rms"] <= MAX_ERR_OVER_RMS, mall
    assert mall["mean_rel_l2"] <= MEAN_REL_L2, mall
