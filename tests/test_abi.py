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

OK, INVALID, MISALIGNED, WORKSPACE = 0, 1, 2, 3
A = 0x10000          # a 256-byte-aligned fake device address
P = ctypes.c_void_p


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
    assert L.moe_workspace_size(64, 32, 4) >= 64 * 4 * 2880 * 2
    assert L.moe_workspace_size(0, 32, 4) > 0
    for T, E, k in [(-1, 32, 4), (4, 32, 0), (4, 32, 9), (4, 3, 4), (4, 257, 4), (1 << 29, 32, 4)]:
        assert L.moe_workspace_size(T, E, k) == 0, (T, E, k)
    # the routed-slot cap: T * k <= 2^22
    assert L.moe_workspace_size(1 << 20, 32, 4) > 0
    assert L.moe_workspace_size((1 << 20) + 1, 32, 4) == 0
    # grows with T and with k
    assert L.moe_workspace_size(128, 32, 4) > L.moe_workspace_size(64, 32, 4)
    assert L.moe_workspace_size(64, 32, 8) > L.moe_workspace_size(64, 32, 4)


def route(L, T=4, E=32, k=4, x=A, Wr=A, br=A, ids=A, w=A, logits=None, ws=A, nbytes=None):
    if nbytes is None:
        nbytes = L.moe_workspace_size(max(T, 0), E, k)
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


def test_pack_validation(L):
    pk = lambda E=2, N=64, c=A, s=A, pc=A, ps=A: L.moe_pack_weights(P(c), P(s), E, N, P(pc), P(ps), None)
    assert pk(E=0) == INVALID
    assert pk(E=257) == INVALID
    assert pk(N=32) == INVALID
    assert pk(N=100) == INVALID
    assert pk(c=None) == INVALID
    assert pk(ps=None) == INVALID
    assert pk(c=A + 8) == MISALIGNED
    assert pk(pc=A + 4) == MISALIGNED
    assert pk(ps=A + 2) == MISALIGNED


def permute(L, T=4, E=32, k=4, ids=A, counts=A, offsets=A, rows=A, ws=A, nbytes=None):
    if nbytes is None:
        nbytes = L.moe_workspace_size(max(T, 0), E, k)
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


def ffn(L, T=4, E=32, k=4, x=A, off=A, rows=A, c13=A, s13=A, b13=A, c2=A, s2=A, b2=A, y=A,
        ws=A, nbytes=None):
    if nbytes is None:
        nbytes = L.moe_workspace_size(max(T, 0), E, k)
    return L.moe_expert_ffn(P(x), P(off), P(rows), P(c13), P(s13), P(b13), P(c2), P(s2), P(b2),
                            T, E, k, P(y), P(ws), nbytes, None)


def test_expert_ffn_validation(L):
    assert ffn(L, T=0) == OK
    assert ffn(L, k=9) == INVALID
    assert ffn(L, c13=None) == INVALID
    assert ffn(L, b2=None) == INVALID
    assert ffn(L, y=None) == INVALID
    assert ffn(L, c13=A + 8) == MISALIGNED
    assert ffn(L, s13=A + 2) == MISALIGNED
    assert ffn(L, c2=A + 1) == MISALIGNED
    assert ffn(L, b13=A + 1) == MISALIGNED
    assert ffn(L, b2=A + 4) == MISALIGNED
    assert ffn(L, y=A + 4) == MISALIGNED
    assert ffn(L, x=A + 2) == MISALIGNED
    assert ffn(L, nbytes=1024) == WORKSPACE


def test_combine_validation(L):
    c = lambda T=4, k=4, y=A, w=A, out=A: L.moe_combine(P(y), P(w), T, k, P(out), None)
    assert c(T=0) == OK
    assert c(T=-1) == INVALID
    assert c(k=0) == INVALID
    assert c(y=None) == INVALID
    assert c(out=A + 4) == MISALIGNED
    assert c(w=A + 2) == MISALIGNED


def fwd(L, T=4, E=32, k=4, x=A, Wr=A, br=A, out=A, ws=A, nbytes=None, c13=A):
    if nbytes is None:
        nbytes = L.moe_workspace_size(max(T, 0), E, k)
    return L.moe_forward(P(x), P(Wr), P(br), P(c13), P(A), P(A), P(A), P(A), P(A),
                         T, E, k, P(out), P(ws), nbytes, None)


def test_forward_validation(L):
    assert fwd(L, T=0) == OK
    assert fwd(L, T=0, x=None, out=None, ws=None) == OK   # T == 0 examines no pointer
    assert fwd(L, T=-1) == INVALID
    assert fwd(L, E=2) == INVALID
    assert fwd(L, x=None) == INVALID
    assert fwd(L, c13=None) == INVALID
    assert fwd(L, out=A + 8) == MISALIGNED
    assert fwd(L, Wr=A + 4) == MISALIGNED
    assert fwd(L, ws=None) == WORKSPACE
    assert fwd(L, nbytes=L.moe_workspace_size(4, 32, 4) - 1) == WORKSPACE


def test_forward_mx6_validation(L):
    def f(T=4, E=32, k=4, x=A, out=A, ws=A, nbytes=None, c13=A):
        if nbytes is None:
            nbytes = L.moe_workspace_size(max(T, 0), E, k)
        return L.moe_forward_mx6(P(x), P(A), P(A), P(c13), P(A), P(A), P(A), P(A), P(A),
                                 T, E, k, P(out), P(ws), nbytes, None)
    assert f(T=0) == OK
    assert f(T=0, x=None, out=None, ws=None) == OK
    assert f(T=-1) == INVALID
    assert f(k=9) == INVALID
    assert f(x=None) == INVALID
    assert f(c13=None) == INVALID
    assert f(out=A + 8) == MISALIGNED
    assert f(ws=None) == WORKSPACE
    # the tiled schedule also holds the activation records in the workspace
    T, E, k = 4096, 32, 4
    assert f(T=T, E=E, k=k, nbytes=L.moe_workspace_size(T, E, k) - 1) == WORKSPACE
    assert L.moe_workspace_size(T, E, k) >= T * 5888 + T * k * 2880 * 6


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
    g = lambda T=4, E=32, k=4, xr=A, off=A, rows=A, c=A, s=A, b=A, h=A: L.moe_gate_up_mx6(
        P(xr), P(off), P(rows), P(c), P(s), P(b), T, E, k, P(h), None)
    assert g(T=0) == OK
    assert g(T=-1) == INVALID
    assert g(xr=None) == INVALID
    assert g(h=None) == INVALID
    assert g(xr=A + 8) == MISALIGNED
    assert g(s=A + 2) == MISALIGNED
    assert g(b=A + 4) == MISALIGNED


def test_forward_block_validation(L):
    def f(T=4, E=32, k=4, x=A, g=A, eps=1e-5, out=A, ws=A, nbytes=None):
        if nbytes is None:
            nbytes = L.moe_workspace_size(max(T, 0), E, k)
        return L.moe_forward_block(P(x), P(g), eps, P(A), P(A), P(A), P(A), P(A), P(A), P(A), P(A),
                                   T, E, k, P(out), P(ws), nbytes, None)
    assert f(T=0) == OK
    assert f(T=-1) == INVALID
    assert f(eps=-1.0) == INVALID
    assert f(eps=float("nan")) == INVALID
    assert f(g=None) == INVALID
    assert f(x=None) == INVALID
    assert f(g=A + 8) == MISALIGNED
    assert f(out=A + 4) == MISALIGNED
    assert f(ws=None) == WORKSPACE
    assert f(nbytes=L.moe_workspace_size(4, 32, 4) - 1) == WORKSPACE


def test_rmsnorm_validation(L):
    n = lambda T=4, x=A, g=A, eps=1e-5, t=A: L.moe_rmsnorm(P(x), P(g), eps, T, P(t), None)
    assert n(T=0) == OK
    assert n(T=-1) == INVALID
    assert n(eps=-0.5) == INVALID
    assert n(x=None) == INVALID
    assert n(t=None) == INVALID
    assert n(g=A + 4) == MISALIGNED
    assert n(t=A + 2) == MISALIGNED
