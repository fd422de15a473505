"""Host checks of the Python binding's validation of caller-supplied outputs.

The kernels write exactly the elements an output's shape implies, densely, so
a mis-sized, mistyped, strided or misplaced output must be refused before the
C call.  These run on CPU tensors against the binding's own check; the GPU
test of the entry points themselves is in test_gpu_binding.py."""
import pytest
import torch

import long_context_attention_dca_amd as dca


def test_output_check_accepts_exact_match():
    t = torch.empty(2, 5, 3, 64)
    dca._check_out(t, "out", (2, 5, 3, 64), torch.float32, "cpu")


@pytest.mark.parametrize("t,exc", [
    (torch.empty(2, 5, 3, 63), ValueError),            # too small: would be written past its end
    (torch.empty(2, 5, 3, 65), ValueError),
    (torch.empty(2, 5, 3), ValueError),
    (torch.empty(2, 5, 3, 64, dtype=torch.bfloat16), TypeError),
    (torch.empty(2, 5, 64, 3).transpose(2, 3), ValueError),   # right shape, not contiguous
    (torch.empty(2, 5, 3, 64, device="meta"), ValueError),    # another device
    ("not a tensor", TypeError),
])
def test_output_check_refuses(t, exc):
    with pytest.raises(exc):
        dca._check_out(t, "out", (2, 5, 3, 64), torch.float32, "cpu")


def test_lse_shape_is_checked_as_float32():
    dca._check_out(torch.empty(1, 4, 10), "lse", (1, 4, 10), torch.float32, "cpu")
    with pytest.raises(ValueError):
        dca._check_out(torch.empty(1, 4, 9), "lse", (1, 4, 10), torch.float32, "cpu")
    with pytest.raises(TypeError):
        dca._check_out(torch.empty(1, 4, 10, dtype=torch.float64), "lse", (1, 4, 10), torch.float32, "cpu")


def test_workspace_check():
    ws = torch.empty(1000, dtype=torch.uint8)
    assert dca._workspace(1000, torch.device("cpu"), ws) is ws
    with pytest.raises(ValueError):
        dca._workspace(1001, torch.device("cpu"), ws)
    with pytest.raises(ValueError):
        dca._workspace(10, torch.device("cpu"), torch.empty(64, dtype=torch.uint8)[::2])
