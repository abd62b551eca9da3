"""ctypes loader of libmoe_mi355x.so and the prototypes of include/moe.h.

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoe_mi355x.so")

# every symbol declared in include/moe.h
EXPORTED = ("moe_workspace_size", "moe_workspace_size_op", "moe_pack_weights", "moe_route", "moe_permute", "moe_expert_ffn",
            "moe_gate_up", "moe_down_accumulate", "moe_combine", "moe_forward",
            "moe_forward_mx6", "moe_encode_mx6", "moe_gate_up_mx6", "moe_forward_block",
            "moe_rmsnorm", "moe_forward_noalloc", "moe_status_string")

MOE_SUCCESS = 0
STATUS_NAMES = {
    0: "MOE_SUCCESS",
    1: "MOE_ERROR_INVALID_VALUE",
    2: "MOE_ERROR_MISALIGNED",
    3: "MOE_ERROR_WORKSPACE",
    4: "MOE_ERROR_UNSUPPORTED",
    5: "MOE_ERROR_HIP",
    6: "MOE_ERROR_LAYOUT",
    7: "MOE_ERROR_RANGE",
}

MOE_PACKED_TAG = 0x3450584D
MOE_NOALLOC_SCRATCH_BYTES = 56 << 20
MOE_MX6_MAX_SCALE_SPREAD = 16

# moe_op_t: the entry points that take a workspace
OPS = {"route": 0, "permute": 1, "expert_ffn": 2, "forward": 3, "forward_mx6": 4,
       "forward_block": 5}


class PackedWeightDesc(ctypes.Structure):
    """moe_packed_weight_t of include/moe.h."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("E", ctypes.c_int32),
                ("N", ctypes.c_int32), ("tag", ctypes.c_uint32), ("scale_spread", ctypes.c_uint32)]

_lib = None


class MoeLibraryMissing(ImportError):
    pass


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoeLibraryMissing(
            f"{LIB_PATH} is missing: build it first (python -m sparse_moe_ffn_fp32_amd.build "
            "or __graft_entry__.build()); the MoE layer has no non-HIP implementation")
    L = ctypes.CDLL(LIB_PATH)
    P, I, SZ, ST = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int
    L.moe_workspace_size.argtypes = [I, I, I]
    L.moe_workspace_size.restype = SZ
    L.moe_workspace_size_op.argtypes = [I, I, I, I]
    L.moe_workspace_size_op.restype = SZ
    L.moe_status_string.argtypes = [ST]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_pack_weights.argtypes = [P, P, I, I, P, P, P, P]
    L.moe_pack_weights.restype = ST
    L.moe_route.argtypes = [P, P, P, I, I, I, P, P, P, P, SZ, P]
    L.moe_route.restype = ST
    L.moe_permute.argtypes = [P, I, I, I, P, P, P, P, SZ, P]
    L.moe_permute.restype = ST
    L.moe_expert_ffn.argtypes = [P, P, P, P, P, P, P, I, I, I, P, P, SZ, P]
    L.moe_expert_ffn.restype = ST
    L.moe_gate_up.argtypes = [P, P, P, P, P, I, I, I, P, P]
    L.moe_gate_up.restype = ST
    L.moe_down_accumulate.argtypes = [P, P, P, P, P, P, I, I, I, P, P]
    L.moe_down_accumulate.restype = ST
    L.moe_combine.argtypes = [P, P, I, I, P, P]
    L.moe_combine.restype = ST
    L.moe_forward.argtypes = [P, P, P, P, P, P, P, I, I, I, P, P, SZ, P]
    L.moe_forward.restype = ST
    L.moe_forward_mx6.argtypes = [P, P, P, P, P, P, P, I, I, I, P, P, SZ, P]
    L.moe_forward_mx6.restype = ST
    L.moe_encode_mx6.argtypes = [P, I, P, P]
    L.moe_encode_mx6.restype = ST
    L.moe_gate_up_mx6.argtypes = [P, P, P, P, P, I, I, I, P, P]
    L.moe_gate_up_mx6.restype = ST
    F = ctypes.c_float
    L.moe_forward_block.argtypes = [P, P, F, P, P, P, P, P, P, I, I, I, P, P, SZ, P]
    L.moe_forward_block.restype = ST
    L.moe_rmsnorm.argtypes = [P, P, F, I, P, P]
    L.moe_rmsnorm.restype = ST
    L.moe_forward_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, P, P]
    L.moe_forward_noalloc.restype = ST
    _lib = L
    return L
