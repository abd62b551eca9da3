"""The C-ABI library without a GPU: it loads, exports every symbol declared in
include/moe.h, and rejects bad arguments on the host before any launch.
No compute call is made here; pointers are fake addresses the library must
never dereference on these paths."""
import ctypes
import os
import re

import pytest

from sparse_moe_ffn_fp32_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, MISALIGNED, WORKSPACE, LAYOUT = 0, 1, 2, 3, 6
A = 0x10000          # a 256-byte-aligned fake device address
P = ctypes.c_void_p
OPS = _native.OPS


def desc(E=32, N=5760, codes=A, scales=A, tag=_native.MOE_PACKED_TAG):
    """A packed-weight descriptor as moe_pack_weights would fill it (fake pointers)."""
    return _native.PackedWeightDesc(codes, scales, E, N, tag, 0)


def dp(d):
    return None if d is None else ctypes.byref(d)


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return _native.lib()


def test_header_symbols_exported(L):
    names = header_functions()
    assert set(names) == set(_native.EXPORTED), names
    for name in names:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in _native.STATUS_NAMES.items():
        assert L.moe_status_string(code).decode().startswith(name)
    assert b"unknown" in L.moe_status_string(99)


def test_workspace_size(L):
    assert L.moe_workspace_size(64, 32, 4) >= 64 * 4 * 2880 * 6
    assert L.moe_workspace_size(0, 32, 4) > 0
    for T, E, k in [(-1, 32, 4), (4, 32, 0), (4, 32, 9), (4, 3, 4), (4, 257, 4), (1 << 29, 32, 4)]:
        assert L.moe_workspace_size(T, E, k) == 0, (T, E, k)
    # the routed-slot cap: T * k <= 2^22
    assert L.moe_workspace_size(1 << 20, 32, 4) > 0
    assert L.moe_workspace_size((1 << 20) + 1, 32, 4) == 0
    # grows with T and with k
    assert L.moe_workspace_size(128, 32, 4) > L.moe_workspace_size(64, 32, 4)
    assert L.moe_workspace_size(64, 32, 8) > L.moe_workspace_size(64, 32, 4)


def test_workspace_size_per_op(L):
    ws = lambda op, T=64, E=32, k=4: L.moe_workspace_size_op(OPS[op], T, E, k)
    T, E, k = 16384, 128, 4
    n = T * k
    # each call asks for what it uses: the router a few MB (its weights split
    # into three bf16 pieces, and the per-32-token expert histograms), not the
    # layer's intermediates
    assert ws("route", T, E, k) <= 3 * 2 * E * 2880 + (T // 32) * E * 4 + 256
    assert ws("permute", T, E, k) <= (T // 32) * E * 4 + 256
    assert ws("permute", 16, 32, 4) == 256            # one workgroup, no scratch
    assert n * 2880 * 2 <= ws("expert_ffn", T, E, k) <= n * 2880 * 2 + 4096
    fwd = ws("forward", T, E, k)
    assert n * 2880 * 6 <= fwd <= n * 2880 * 6 + 16 * n + ws("route", T, E, k) + 8192
    # the FP6 records only for moe_forward_mx6, the normed input only for the block
    assert ws("forward_mx6", T, E, k) >= fwd + (T + n) * 5888
    assert ws("forward_block", T, E, k) >= fwd + T * 2880 * 2
    assert ws("forward_block", T, E, k) < ws("forward_mx6", T, E, k)
    # decode sizes: the router forms the inverse RMS itself (no buffer for
    # it), only the normed rows are added
    assert ws("forward_block", 64, 32, 4) == ws("forward", 64, 32, 4) + 64 * 2880 * 2
    # decode sizes: no records (weight-streaming schedule)
    assert ws("forward_mx6", 64, 32, 4) == ws("forward", 64, 32, 4)
    # the all-ops size is the largest
    for T, E, k in [(1, 8, 2), (64, 32, 4), (4096, 32, 4), (T, E, k)]:
        assert L.moe_workspace_size(T, E, k) == max(L.moe_workspace_size_op(o, T, E, k) for o in OPS.values())
    assert L.moe_workspace_size_op(6, 64, 32, 4) == 0
    assert L.moe_workspace_size_op(-1, 64, 32, 4) == 0
    assert L.moe_workspace_size_op(OPS["forward"], 64, 3, 4) == 0


def route(L, T=4, E=32, k=4, x=A, Wr=A, br=A, ids=A, w=A, logits=None, ws=A, nbytes=None):
    if nbytes is None:
        nbytes = L.moe_workspace_size_op(OPS["route"], max(T, 0), E, k)
    return L.moe_route(P(x), P(Wr), P(br), T, E, k, P(ids), P(w), P(logits), P(ws), nbytes, None)


def test_route_validation(L):
    assert route(L, T=0) == OK
    assert route(L, T=-1) == INVALID
    assert route(L, k=0) == INVALID
    assert route(L, k=9) == INVALID
    assert route(L, E=3) == INVALID
    assert route(L, E=300) == INVALID
    assert route(L, x=None) == INVALID
    assert route(L, Wr=None) == INVALID
    assert route(L, w=None) == INVALID
    assert route(L, x=A + 8) == MISALIGNED
    assert route(L, Wr=A + 4) == MISALIGNED
    assert route(L, ids=A + 2) == MISALIGNED
    assert route(L, logits=A + 1) == MISALIGNED
    assert route(L, ws=None) == WORKSPACE
    assert route(L, nbytes=64) == WORKSPACE
    assert route(L, nbytes=L.moe_workspace_size_op(OPS["route"], 4, 32, 4) - 1) == WORKSPACE


def test_pack_validation(L):
    out = desc(tag=0)
    pk = lambda E=2, N=64, c=A, s=A, pc=A, ps=A, d=out: L.moe_pack_weights(
        P(c), P(s), E, N, P(pc), P(ps), dp(d), None)
    assert pk(E=0) == INVALID
    assert pk(E=257) == INVALID
    assert pk(N=32) == INVALID
    assert pk(N=100) == INVALID
    assert pk(c=None) == INVALID
    assert pk(ps=None) == INVALID
    assert pk(c=A + 8) == MISALIGNED
    assert pk(pc=A + 4) == MISALIGNED
    assert pk(ps=A + 2) == MISALIGNED
    assert pk(d=None) == INVALID
    assert out.tag == 0      # a refused call leaves the descriptor alone


def permute(L, T=4, E=32, k=4, ids=A, counts=A, offsets=A, rows=A, ws=A, nbytes=None):
    if nbytes is None:
        nbytes = L.moe_workspace_size_op(OPS["permute"], max(T, 0), E, k)
    return L.moe_permute(P(ids), T, E, k, P(counts), P(offsets), P(rows), P(ws), nbytes, None)


def test_permute_validation(L):
    assert permute(L, T=0) == OK
    assert permute(L, T=-3) == INVALID
    assert permute(L, ids=None) == INVALID
    assert permute(L, rows=None) == INVALID
    assert permute(L, offsets=A + 2) == MISALIGNED
    assert permute(L, ws=None) == WORKSPACE
    assert permute(L, ws=A + 16) == WORKSPACE
    assert permute(L, nbytes=16) == WORKSPACE
    T, E, k = 4096, 32, 4
    need = L.moe_workspace_size_op(OPS["permute"], T, E, k)
    assert permute(L, T=T, E=E, k=k, nbytes=need - 1) == WORKSPACE


def ffn(L, T=4, E=32, k=4, x=A, off=A, rows=A, w13="d", b13=A, w2="d", b2=A, y=A,
        ws=A, nbytes=None):
    if nbytes is None:
        nbytes = L.moe_workspace_size_op(OPS["expert_ffn"], max(T, 0), E, k)
    w13 = desc(E, 5760) if w13 == "d" else w13
    w2 = desc(E, 2880) if w2 == "d" else w2
    return L.moe_expert_ffn(P(x), P(off), P(rows), dp(w13), P(b13), dp(w2), P(b2),
                            T, E, k, P(y), P(ws), nbytes, None)


def test_expert_ffn_validation(L):
    assert ffn(L, T=0) == OK
    assert ffn(L, k=9) == INVALID
    assert ffn(L, w13=None) == INVALID
    assert ffn(L, b2=None) == INVALID
    assert ffn(L, y=None) == INVALID
    assert ffn(L, w13=desc(codes=A + 8)) == MISALIGNED
    assert ffn(L, w13=desc(scales=A + 2)) == MISALIGNED
    assert ffn(L, w2=desc(N=2880, codes=A + 1)) == MISALIGNED
    assert ffn(L, b13=A + 1) == MISALIGNED
    assert ffn(L, b2=A + 4) == MISALIGNED
    assert ffn(L, y=A + 4) == MISALIGNED
    assert ffn(L, x=A + 2) == MISALIGNED
    assert ffn(L, nbytes=1024) == WORKSPACE


def test_packed_descriptor_required(L):
    """Weights reach the GEMMs only through a descriptor that moe_pack_weights
    tagged, with the call's expert count and row count."""
    assert ffn(L, w13=desc(tag=0)) == LAYOUT                  # never packed
    assert ffn(L, w13=desc(tag=_native.MOE_PACKED_TAG ^ 1)) == LAYOUT
    assert ffn(L, w13=desc(N=2880)) == LAYOUT                 # the down tensor as gate/up
    assert ffn(L, w2=desc(N=5760)) == LAYOUT                  # the gate/up tensor as down
    assert ffn(L, w13=desc(E=16)) == LAYOUT                   # other expert count
    assert ffn(L, w2=desc(E=31, N=2880)) == LAYOUT
    assert ffn(L, w13=desc(codes=None)) == LAYOUT
    g = lambda w: L.moe_gate_up(P(A), P(A), P(A), dp(w), P(A), 4, 32, 4, P(A), None)
    assert g(desc(tag=0)) == LAYOUT
    assert g(desc(N=2880)) == LAYOUT
    assert g(None) == INVALID
    da = lambda w: L.moe_down_accumulate(P(A), P(A), P(A), P(A), dp(w), P(A), 4, 32, 4, P(A), None)
    assert da(desc(N=5760)) == LAYOUT
    assert da(desc(tag=0, N=2880)) == LAYOUT
    for fn in (L.moe_forward, L.moe_forward_mx6):
        f = lambda w13, w2: fn(P(A), P(A), P(A), dp(w13), P(A), dp(w2), P(A), 4, 32, 4, P(A), P(A),
                               L.moe_workspace_size(4, 32, 4), None)
        assert f(desc(tag=0), desc(N=2880)) == LAYOUT
        assert f(desc(), desc(N=2880, tag=0)) == LAYOUT
        assert f(desc(), desc()) == LAYOUT                     # w2 with 5760 rows
        assert f(desc(E=128), desc(E=128, N=2880)) == LAYOUT   # router has 32 experts


def test_combine_validation(L):
    c = lambda T=4, k=4, y=A, w=A, out=A: L.moe_combine(P(y), P(w), T, k, P(out), None)
    assert c(T=0) == OK
    assert c(T=-1) == INVALID
    assert c(k=0) == INVALID
    assert c(y=None) == INVALID
    assert c(out=A + 4) == MISALIGNED
    assert c(w=A + 2) == MISALIGNED


def fwd(L, T=4, E=32, k=4, x=A, Wr=A, br=A, out=A, ws=A, nbytes=None, w13="d"):
    if nbytes is None:
        nbytes = L.moe_workspace_size_op(OPS["forward"], max(T, 0), E, k)
    w13 = desc(E, 5760) if w13 == "d" else w13
    return L.moe_forward(P(x), P(Wr), P(br), dp(w13), P(A), dp(desc(E, 2880)), P(A),
                         T, E, k, P(out), P(ws), nbytes, None)


def test_forward_validation(L):
    assert fwd(L, T=0) == OK
    assert fwd(L, T=0, x=None, out=None, ws=None) == OK   # T == 0 examines no pointer
    assert fwd(L, T=-1) == INVALID
    assert fwd(L, E=2) == INVALID
    assert fwd(L, x=None) == INVALID
    assert fwd(L, w13=None) == INVALID
    assert fwd(L, out=A + 8) == MISALIGNED
    assert fwd(L, Wr=A + 4) == MISALIGNED
    assert fwd(L, ws=None) == WORKSPACE
    assert fwd(L, nbytes=L.moe_workspace_size_op(OPS["forward"], 4, 32, 4) - 1) == WORKSPACE


def test_forward_mx6_validation(L):
    def f(T=4, E=32, k=4, x=A, out=A, ws=A, nbytes=None, w13="d"):
        if nbytes is None:
            nbytes = L.moe_workspace_size_op(OPS["forward_mx6"], max(T, 0), E, k)
        w13 = desc(E, 5760) if w13 == "d" else w13
        return L.moe_forward_mx6(P(x), P(A), P(A), dp(w13), P(A), dp(desc(E, 2880)), P(A),
                                 T, E, k, P(out), P(ws), nbytes, None)
    assert f(T=0) == OK
    assert f(T=0, x=None, out=None, ws=None) == OK
    assert f(T=-1) == INVALID
    assert f(k=9) == INVALID
    assert f(x=None) == INVALID
    assert f(w13=None) == INVALID
    assert f(out=A + 8) == MISALIGNED
    assert f(ws=None) == WORKSPACE
    # the tiled schedule also holds the activation records in the workspace
    T, E, k = 4096, 32, 4
    need = L.moe_workspace_size_op(OPS["forward_mx6"], T, E, k)
    assert f(T=T, E=E, k=k, nbytes=need - 1) == WORKSPACE
    assert need >= T * 5888 + T * k * 2880 * 6


def test_encode_mx6_validation(L):
    enc = lambda rows=4, x=A, rec=A: L.moe_encode_mx6(P(x), rows, P(rec), None)
    assert enc(rows=0) == OK
    assert enc(rows=0, x=None, rec=None) == OK
    assert enc(rows=-1) == INVALID
    assert enc(rows=(1 << 22) + 1) == INVALID
    assert enc(x=None) == INVALID
    assert enc(rec=None) == INVALID
    assert enc(x=A + 8) == MISALIGNED
    assert enc(rec=A + 4) == MISALIGNED


def test_gate_up_mx6_validation(L):
    g = lambda T=4, E=32, k=4, xr=A, off=A, rows=A, w="d", b=A, h=A: L.moe_gate_up_mx6(
        P(xr), P(off), P(rows), dp(desc(E, 5760) if w == "d" else w), P(b), T, E, k, P(h), None)
    assert g(T=0) == OK
    assert g(T=-1) == INVALID
    assert g(xr=None) == INVALID
    assert g(h=None) == INVALID
    assert g(w=None) == INVALID
    assert g(xr=A + 8) == MISALIGNED
    assert g(w=desc(scales=A + 2)) == MISALIGNED
    assert g(b=A + 4) == MISALIGNED
    assert g(w=desc(tag=0)) == LAYOUT


def test_forward_block_validation(L):
    def f(T=4, E=32, k=4, x=A, g=A, eps=1e-5, out=A, ws=A, nbytes=None):
        if nbytes is None:
            nbytes = L.moe_workspace_size_op(OPS["forward_block"], max(T, 0), E, k)
        return L.moe_forward_block(P(x), P(g), eps, P(A), P(A), dp(desc(E, 5760)), P(A),
                                   dp(desc(E, 2880)), P(A), T, E, k, P(out), P(ws), nbytes, None)
    assert f(T=0) == OK
    assert f(T=-1) == INVALID
    assert f(eps=-1.0) == INVALID
    assert f(eps=float("nan")) == INVALID
    assert f(g=None) == INVALID
    assert f(x=None) == INVALID
    assert f(g=A + 8) == MISALIGNED
    assert f(out=A + 4) == MISALIGNED
    assert f(ws=None) == WORKSPACE
    assert f(nbytes=L.moe_workspace_size_op(OPS["forward_block"], 4, 32, 4) - 1) == WORKSPACE


def test_rmsnorm_validation(L):
    n = lambda T=4, x=A, g=A, eps=1e-5, t=A: L.moe_rmsnorm(P(x), P(g), eps, T, P(t), None)
    assert n(T=0) == OK
    assert n(T=-1) == INVALID
    assert n(eps=-0.5) == INVALID
    assert n(x=None) == INVALID
    assert n(t=None) == INVALID
    assert n(g=A + 4) == MISALIGNED
    assert n(t=A + 2) == MISALIGNED


def test_forward_noalloc_validation(L):
    """The allocation-free layer: argument checks as moe_forward, and sizes
    whose workspace exceeds the library's scratch refused before any launch."""
    def f(T=4, E=32, k=4, x=A, out=A, w13="d"):
        w13 = desc(E, 5760) if w13 == "d" else w13
        return L.moe_forward_noalloc(P(x), P(A), P(A), dp(w13), P(A), dp(desc(E, 2880)), P(A),
                                     T, E, k, P(out), None)
    assert f(T=0) == OK
    assert f(T=0, x=None, out=None) == OK
    assert f(T=-1) == INVALID
    assert f(k=9) == INVALID
    assert f(x=None) == INVALID
    assert f(out=None) == INVALID
    assert f(w13=None) == INVALID
    assert f(w13=desc(tag=0)) == LAYOUT
    assert f(out=A + 8) == MISALIGNED
    cap = _native.MOE_NOALLOC_SCRATCH_BYTES
    big = next(T for T in range(512, 4096, 8) if L.moe_workspace_size_op(OPS["forward"], T, 32, 4) > cap)
    assert f(T=big) == WORKSPACE
    assert L.moe_workspace_size_op(OPS["forward"], big - 8, 32, 4) <= cap
