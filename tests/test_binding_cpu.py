"""CPU checks of the Python binding's buffer validation: the C library cannot see
buffer sizes, so the binding rejects host tensors, short buffers, wrong dtypes and
non-contiguous buffers before anything is launched."""

import pytest
import torch

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import _buf, _OUT_DTYPES, _out, _U8, _I32

CPU = torch.device("cpu")


def test_buf_accepts_a_matching_buffer():
    t = torch.zeros(64, dtype=torch.uint8)
    assert _buf(t, "q", _U8, 64, CPU) is t


@pytest.mark.parametrize("t,err", [
    (torch.zeros(63, dtype=torch.uint8), ValueError),  # too short
    (torch.zeros(64, dtype=torch.int8), TypeError),  # dtype
    (torch.zeros(8, 16, dtype=torch.uint8).t(), ValueError),  # not contiguous
    ([0] * 64, TypeError),  # not a tensor
])
def test_buf_rejects(t, err):
    with pytest.raises(err):
        _buf(t, "q", _U8, 64, CPU)


def test_buf_rejects_another_device():
    with pytest.raises(ValueError):
        _buf(torch.zeros(4, dtype=torch.int32), "offs", _I32, 4, torch.device("cuda:0"))


def test_out_dtype_must_match():
    # an fp32 output request with a bf16 buffer would be written with twice its bytes
    with pytest.raises(TypeError):
        _out((4, 4), mx.MX_OUT_F32, CPU, torch.zeros(4, 4, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        _out((4, 4), mx.MX_OUT_BF16, CPU, torch.zeros(4, 4, dtype=torch.float32))
    with pytest.raises(ValueError):
        _out((4, 4), mx.MX_OUT_F32, CPU, torch.zeros(15, dtype=torch.float32))
    with pytest.raises(ValueError):
        _out((4, 4), 7, CPU, None)
    assert _OUT_DTYPES[mx.MX_OUT_F32] == (torch.float32,)


def test_gemm_calls_reject_host_tensors():
    a = torch.zeros(64, 64, dtype=torch.uint8)
    s = torch.zeros(mx.mx_scale_bytes(64, 64), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU memory"):
        mx.mx_grouped_mm_fwd(a, s, a, s, None, 64, 64, 64)
    with pytest.raises(ValueError, match="GPU memory"):
        mx.mx_grouped_mm_wgrad(a, s, a, s, None, 64, 64, 64)
    with pytest.raises(ValueError, match="GPU memory"):
        mx.mx_quantize_dim0(torch.zeros(32, 64, dtype=torch.bfloat16))


def test_workspace_query():
    assert mx.mx_grouped_mm_wgrad_workspace_bytes(1, 16384, 576, 4096) == 5 * 576 * 4096 * 4
    assert mx.mx_grouped_mm_wgrad_workspace_bytes(8, 16384, 4096, 4096) == 0
    with pytest.raises(ValueError):
        mx.mx_grouped_mm_wgrad_workspace_bytes(0, 16384, 4096, 4096)


def test_binding_has_every_entry_point():
    """The binding carries the C ABI's names: every function the header declares."""
    import re
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    text = open(os.path.join(here, "..", "include", "mxfp8.h")).read()
    names = sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))
    assert names and not [n for n in names if not hasattr(mx, n)]
    assert mx.mx_status_string(0) == "MX_OK"
    assert mx.mx_status_string(-2) == "MX_E_SHAPE"


def test_pad_quantize_ex_flags():
    x = torch.zeros(64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mx.mx_pad_quantize_ex(x, torch.tensor([64], dtype=torch.int32), flags=1)
