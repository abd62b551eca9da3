"""Host-side checks of the Python binding (no GPU needed)."""
import pytest
import torch

import sparse_moe_ffn_fp32_amd as moe


def test_one_device_per_call():
    # the device check runs before any stream or kernel is touched
    a = torch.empty(4, device="meta")
    b = torch.empty(4)
    with pytest.raises(ValueError, match="one device"):
        moe._stream(a, b)
    with pytest.raises(ValueError, match="one device"):
        moe._stream(a, None, b)


def test_host_tensors_rejected():
    x = torch.zeros((2, 2880), dtype=torch.int16)
    with pytest.raises(ValueError, match="GPU device"):
        moe.encode_mx6(x)


def test_unpacked_weights_rejected():
    """The layer calls take the expert weights only as a PackedExperts: the
    checkpoint-layout tensors (or the old flat argument list) raise before any
    device work."""
    codes = torch.zeros((2, 5760, 1440), dtype=torch.uint8)
    with pytest.raises(TypeError, match="PackedExperts"):
        moe._experts(codes)
    with pytest.raises(TypeError, match="PackedExperts"):
        moe._experts((codes, codes))
    x = torch.zeros((1, 2880), dtype=torch.int16)
    with pytest.raises(TypeError):
        # nine weight tensors where one PackedExperts belongs
        moe.forward(x, x, x, codes, codes, x, codes, codes, x, 4)


def test_workspace_ops_named():
    assert set(moe._native.OPS) == {"route", "permute", "expert_ffn", "forward", "forward_mx6",
                                    "forward_block"}
