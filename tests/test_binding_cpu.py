"""Host-side argument checks of the Python binding: caller-supplied outputs
and scratch buffers are validated before their addresses reach the library,
which writes through them without knowing their extent (no GPU needed)."""
import pytest
import torch

from activation_sparse_ffn_amd import _need_buffer


def test_need_buffer_accepts_a_matching_tensor():
    _need_buffer(torch.empty(4, 8), "y", (4, 8), torch.float32, torch.device("cpu"))
    _need_buffer(torch.empty(100, dtype=torch.uint8), "workspace", None, torch.uint8, torch.device("cpu"))


@pytest.mark.parametrize("t,shape,dtype,what", [
    (torch.empty(4, 7), (4, 8), torch.float32, "shape"),
    (torch.empty(5, 8), (4, 8), torch.float32, "shape"),
    (torch.empty(4, 8, dtype=torch.float64), (4, 8), torch.float32, "float32"),
    (torch.empty(4, 8, dtype=torch.int32), (4, 8), torch.int64, "int64"),
    (torch.empty(8, 4).t(), (4, 8), torch.float32, "contiguous"),
])
def test_need_buffer_rejects(t, shape, dtype, what):
    with pytest.raises(ValueError, match=what):
        _need_buffer(t, "out", shape, dtype, torch.device("cpu"))


def test_need_buffer_rejects_another_device():
    with pytest.raises(ValueError, match="meta"):
        _need_buffer(torch.empty(4, 8, device="meta"), "y", (4, 8), torch.float32, torch.device("cpu"))
    with pytest.raises(TypeError):
        _need_buffer(None, "y", (4, 8), torch.float32, torch.device("cpu"))
