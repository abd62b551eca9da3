"""Shared helpers of the GPU parity tests: host -> device transfer, the
acceptance metrics (max error over RMS, mean per-token relative L2), and the near-tie rule for routing."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Pass criteria of the layer output (max error relative to the reference RMS,
# and mean over tokens of the per-token relative L2 error).
MAX_ERR_OVER_RMS = 2e-2
MEAN_REL_L2 = 5e-3
# Tokens whose k-th / (k+1)-th oracle logit gap is below this may pick a
# different expert set.
NEAR_TIE_GAP = 1e-4


def to_device(inp, device="cuda", pack=True):
    """Host arrays -> device tensors; with `pack`, the expert weights are also
    packed on the GPU (key "experts", a PackedExperts)."""
    import sparse_moe_ffn_fp32_amd as moe
    d = {}
    for key, a in inp.items():
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        d[key] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    if pack and "w13_codes" in d:
        d["experts"] = moe.pack_experts(d["w13_codes"], d["w13_scales"], d["b13"],
                                        d["w2_codes"], d["w2_scales"], d["b2"])
    return d


def weights_args(d):
    """The packed expert weights, as the layer calls take them."""
    return (d["experts"],)


def pack_reference(codes: np.ndarray, scales: np.ndarray):
    """The documented packed order, written independently of the library:
    offset(codes) = G*92160 + s*4096 + m*(s < 22 ? 1024 : 512) + l*16,
    offset(scales) = G*5760 + s*256 + l*4 + m, for row 64G + 16m + r,
    MX block 4s + g, lane l = 16g + r."""
    E, N, _ = codes.shape
    pc = np.zeros(E * N * 1440, dtype=np.uint8)
    ps = np.zeros(E * N * 90, dtype=np.uint8)
    rows = np.arange(E * N)
    G, rin = rows // 64, rows % 64
    m, r = rin // 16, rin % 16
    cflat = codes.reshape(E * N, 90, 16)
    sflat = scales.reshape(E * N, 90)
    for kb in range(90):
        s, g = kb // 4, kb % 4
        l = 16 * g + r
        off = G * 92160 + s * 4096 + m * (1024 if s < 22 else 512) + l * 16
        pc[off[:, None] + np.arange(16)[None, :]] = cflat[:, kb, :]
        ps[G * 5760 + s * 256 + l * 4 + m] = sflat[:, kb]
    return pc.reshape(codes.shape), ps.reshape(scales.shape)


def out_metrics(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    err = got - ref
    rms = float(np.sqrt(np.mean(ref ** 2)))
    max_rel = float(np.max(np.abs(err)) / rms) if rms > 0 else float(np.max(np.abs(err)))
    nt = np.linalg.norm(ref, axis=1)
    per_tok = np.linalg.norm(err, axis=1) / np.where(nt > 0, nt, 1.0)
    return dict(max_err_over_rms=max_rel, mean_rel_l2=float(per_tok.mean()),
                global_rel_l2=float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)),
                finite=bool(np.all(np.isfinite(got))))


def assert_out_close(got, ref, label=""):
    m = out_metrics(got, ref)
    assert m["finite"], f"{label}: non-finite output"
    assert m["max_err_over_rms"] <= MAX_ERR_OVER_RMS, (label, m)
    assert m["mean_rel_l2"] <= MEAN_REL_L2, (label, m)
    return m


def check_routing(ids_gpu, w_gpu, logits64, k):
    """Top-k sets must match the float64 oracle except on near-tie tokens.
    Returns the GPU ids (for the oracle to follow on excluded tokens) and the
    number of near-tie tokens whose set differed."""
    ids_ref, gap = oracle.select_topk(logits64, k)
    same = np.array([set(a) == set(b) for a, b in zip(ids_gpu.tolist(), ids_ref.tolist())])
    bad = ~same & (gap >= NEAR_TIE_GAP)
    assert not bad.any(), f"expert sets differ on {int(bad.sum())} tokens with gap >= {NEAR_TIE_GAP}"
    # within a token: distinct experts, descending logits
    T = ids_gpu.shape[0]
    for t in range(T):
        assert len(set(ids_gpu[t].tolist())) == k
    sel = np.take_along_axis(logits64, ids_gpu.astype(np.int64), axis=1)
    assert np.all(np.diff(sel, axis=1) <= 2e-5)
    # weights: softmax of the float64 logits of the GPU's own set
    w_ref = oracle.routing_weights(logits64, ids_gpu.astype(np.int64))
    assert np.max(np.abs(w_gpu - w_ref)) < 2e-5, np.max(np.abs(w_gpu - w_ref))
    return int((~same).sum())


def expert_edge_tokens(ids: np.ndarray, E: int) -> np.ndarray:
    """The tokens that own each expert's first and last routed slot (slot
    order t*k + j): with the stable expert-sorted order these are the first
    and last rows of every expert's range, so its first tile and its ragged
    last tile are both checked."""
    flat = np.asarray(ids).reshape(-1)
    k = ids.shape[1]
    toks = []
    for e in range(E):
        where = np.nonzero(flat == e)[0]
        if where.size:
            toks += [where[0] // k, where[-1] // k]
    return np.unique(np.asarray(toks, dtype=np.int64))


def oracle_for_gpu_routing(inp, k, ref, ids_gpu, T):
    """Oracle outputs (out [T, H] and per-slot y [T, k, H] in the GPU's slot
    order) for the first T tokens of `inp`, from one shared oracle run `ref`
    (oracle.forward(inp, k, keep_y=True) over all tokens). Tokens whose GPU
    expert set differs from the oracle's (near ties only, checked by
    check_routing) are recomputed with the GPU's set."""
    ids_ref = ref["ids"][:T]
    out = ref["out"][:T].copy()
    y = np.empty((T, k, ref["y"].shape[2]), dtype=np.float64)
    redo = []
    for t in range(T):
        if set(ids_gpu[t].tolist()) != set(ids_ref[t].tolist()):
            redo.append(t)
            continue
        pos = {int(e): j for j, e in enumerate(ids_ref[t])}
        for j in range(k):
            y[t, j] = ref["y"][t, pos[int(ids_gpu[t, j])]]
    if redo:
        full = np.array(ref["ids"])
        full[:T] = ids_gpu
        r2 = oracle.forward(inp, k, tokens=np.asarray(redo), ids_override=full, keep_y=True)
        out[redo] = r2["out"]
        y[redo] = r2["y"]
    return out, y


_ORACLE_CASES = {}


def oracle_case(T, E, k, seed):
    """(inputs, oracle.forward(inputs, k, keep_y=True)) of make_layer_inputs(T,
    E, k, seed), computed once per process for the most recent key (large
    cases are shared between test modules)."""
    from moe_inputs import make_layer_inputs
    key = (T, E, k, seed)
    if key not in _ORACLE_CASES:
        _ORACLE_CASES.clear()
        inp = make_layer_inputs(T, E, k, seed=seed)
        _ORACLE_CASES[key] = (inp, oracle.forward(inp, k, keep_y=True))
    return _ORACLE_CASES[key]
