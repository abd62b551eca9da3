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
