"""The C-ABI library loads, exports every declared entry point and validates its
arguments on the host (no GPU needed: nothing here launches a kernel)."""

import os
import re

import pytest

from mxfp8_block_scaled_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")

MX_E_NULL, MX_E_SHAPE, MX_E_ALIGN, MX_E_LAYOUT, MX_E_DTYPE, MX_E_DEVICE = -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_instrumented_build_is_separate(lib):
    # the product library carries no cycle-stamp code; the instrumented copy exports
    # the same entry points plus its record reader
    import ctypes

    from mxfp8_block_scaled_amd import build

    assert not hasattr(lib, "mx_cycle_stamps_read")
    if not os.path.exists(build.STAMPS_LIB):
        pytest.skip("instrumented library not built")
    st = ctypes.CDLL(build.STAMPS_LIB)
    for n in declared_functions() + ["mx_cycle_stamps_blocks", "mx_cycle_stamps_read", "mx_cycle_stamps_clear"]:
        assert hasattr(st, n), n
    st.mx_cycle_stamps_blocks.restype = ctypes.c_int64
    assert st.mx_cycle_stamps_blocks() == 32768


def test_scale_bytes(lib):
    assert lib.mx_scale_bytes(32, 256) == 256
    assert lib.mx_scale_bytes(33, 256) == 512
    assert lib.mx_scale_bytes(32, 288) == 512
    assert lib.mx_scale_bytes(576, 4096) == 18 * 16 * 256
    assert lib.mx_scale_bytes(0, 64) == 0
    assert lib.mx_scale_bytes(32, 48) == -1
    assert lib.mx_scale_bytes(-1, 32) == -1


def test_status_strings(lib):
    assert lib.mx_status_string(0) == b"MX_OK"
    assert lib.mx_status_string(-2) == b"MX_E_SHAPE"
    assert lib.mx_status_string(-99) == b"MX_E_UNKNOWN"


# fake, aligned, never dereferenced device addresses: validation fails before any launch
P = 0x10000
P2 = 0x20000


@pytest.mark.parametrize(
    "args,status",
    [
        ((P, 4, 48, 48, P2, P2, None), MX_E_SHAPE),  # cols not a multiple of 32
        ((P, -1, 32, 32, P2, P2, None), MX_E_SHAPE),
        ((P, 4, 64, 32, P2, P2, None), MX_E_LAYOUT),  # pitch < cols
        ((P, 4, 64, 68, P2, P2, None), MX_E_ALIGN),  # pitch breaks 16-byte rows
        ((None, 4, 64, 64, P2, P2, None), MX_E_NULL),
        ((P + 2, 4, 64, 64, P2, P2, None), MX_E_ALIGN),
        ((P, 4, 64, 64, P2, None, None), MX_E_NULL),
    ],
)
def test_dim0_validation(lib, args, status):
    assert lib.mx_quantize_dim0(*args) == status
    assert len(lib.mx_last_error()) > 0


def test_dim0_dim1_validation(lib):
    f = lib.mx_quantize_dim0_dim1
    assert f(P, 1, 48, 64, 64, P2, P2, P2, P2, None) == MX_E_SHAPE  # rows % 32
    assert f(P, 1, 64, 48, 64, P2, P2, P2, P2, None) == MX_E_SHAPE  # cols % 32
    assert f(P, 0, 64, 64, 64, P2, P2, P2, P2, None) == MX_E_SHAPE  # batch
    assert f(P, 1, 64, 64, 32, P2, P2, P2, P2, None) == MX_E_LAYOUT  # pitch < cols
    assert f(P, 1, 64, 64, 64, P2, P2, None, P2, None) == MX_E_NULL  # q_t
    assert f(P, 1, 64, 64, 64, P2, P2, P2, None, None) == MX_E_NULL  # scale_t
    assert f(P, 1, 64, 64, 64, P2 + 4, P2, P2, P2, None) == MX_E_ALIGN
    # the one-pass cast's 32-bit buffer offsets: row pitch below 2^25, rows below 2^29
    assert f(P, 1, 64, 64, 1 << 25, P2, P2, P2, P2, None) == MX_E_SHAPE
    assert f(P, 1, 1 << 29, 32, 32, P2, P2, P2, P2, None) == MX_E_SHAPE
    assert lib.mx_quantize_ex(P, 1, 64, 64, 1 << 25, 3, 0, P2, P2, P2, P2, None) == MX_E_SHAPE
    assert lib.mx_quantize_ex(P, 1, 64, 64, 1 << 25, 1, 0, P2, P2, None, None, None) in (MX_E_DEVICE, 0)


def test_quantize_ex_validation(lib):
    f = lib.mx_quantize_ex
    assert f(P, 1, 64, 64, 64, 0, 0, P2, P2, P2, P2, None) == MX_E_DTYPE  # no form
    assert f(P, 1, 64, 64, 64, 4, 0, P2, P2, P2, P2, None) == MX_E_DTYPE  # unknown form
    assert f(P, 1, 64, 64, 64, 3, 2, P2, P2, P2, P2, None) == MX_E_DTYPE  # unknown scale rule
    assert f(P, 1, 64, 64, 64, 2 | 4, 0, None, None, P2, P2, None) == MX_E_DTYPE  # stream hint needs both forms
    assert f(P, 1, 64, 64, 64, 8 | 3, 0, P2, P2, P2, P2, None) == MX_E_DTYPE  # unknown bit
    assert f(P, 1, 64, 64, 64, 3 | 4, 0, P2, P2, P2, P2, None) in (MX_E_DEVICE, 0)  # one-pass with the hint
    assert f(P, 1, 48, 64, 64, 2, 1, None, None, P2, P2, None) == MX_E_SHAPE  # dim1 needs rows % 32
    assert f(P, 1, 48, 64, 64, 1, 1, P2, P2, None, None, None) in (MX_E_DEVICE, 0)  # dim0 alone: any rows
    assert f(P, 1, 64, 64, 64, 1, 1, None, P2, None, None, None) == MX_E_NULL  # dim0 output missing
    assert f(P, 1, 64, 64, 64, 3, 1, P2, P2, None, P2, None) == MX_E_NULL  # dim1 output missing


def test_dim1_and_w32_validation(lib):
    assert lib.mx_quantize_dim1(P, 1, 48, 64, 64, P2, P2, None) == MX_E_SHAPE  # rows % 32
    assert lib.mx_quantize_dim1(P, 0, 64, 64, 64, P2, P2, None) == MX_E_SHAPE  # batch
    assert lib.mx_quantize_weight_32x32(P, 1, 40, 64, 64, P2, None, P2, None, None) == MX_E_SHAPE
    assert lib.mx_quantize_weight_32x32(P, 1, 64, 64, 64, P2, P2, P2, None, None) == MX_E_NULL  # q_t without scale_col


def test_gemm_validation(lib):
    f = lib.mx_grouped_mm_fwd
    assert f(P, P, P, P, None, 1, 64, 64, 48, P2, 0, None) == MX_E_SHAPE  # k % 32
    assert f(P, P, P, P, None, 2, 64, 64, 64, P2, 0, None) == MX_E_SHAPE  # dense with groups > 1
    assert f(P, P, P, P, P, 2, 64, 40, 64, P2, 0, None) == MX_E_SHAPE  # grouped n % 32
    assert f(P, P, P, P, None, 1, 64, 64, 64, P2, 7, None) == MX_E_DTYPE
    assert f(P, P, P, P, P + 2, 1, 64, 64, 64, P2, 0, None) == MX_E_ALIGN
    assert lib.mx_grouped_mm_dgrad(P, P, P, P, None, 1, 64, 40, 64, P2, 0, None) == MX_E_SHAPE  # n % 32
    assert lib.mx_grouped_mm_wgrad(P, P, P, P, None, 1, 40, 64, 64, P2, 0, None, 0, None) == MX_E_SHAPE  # m % 32
    # extent limits: contraction above 2^22, or a scale buffer reaching 2^31 bytes
    big = (1 << 22) + 32
    assert f(P, P, P, P, None, 1, 64, 64, big, P2, 0, None) == MX_E_SHAPE
    assert b"2^22" in lib.mx_last_error()
    assert lib.mx_grouped_mm_dgrad(P, P, P, P, None, 1, 64, big, 64, P2, 0, None) == MX_E_SHAPE
    assert lib.mx_grouped_mm_wgrad(P, P, P, P, None, 1, big, 64, 64, P2, 0, None, 0, None) == MX_E_SHAPE
    assert f(P, P, P, P, None, 1, 1 << 30, 64, 1 << 22, P2, 0, None) == MX_E_SHAPE  # a's scales: 2^47 bytes
    assert b"2^31" in lib.mx_last_error()
    assert lib.mx_grouped_mm_wgrad(P, P, P, P, None, 1, 1 << 22, 1 << 16, 64, P2, 0, None, 0, None) == MX_E_SHAPE  # 2^33
    # at the limit the shapes are accepted (no GPU here: the device check answers)
    assert f(P, P, P, P, None, 1, 64, 64, 1 << 22, P2, 0, None) in (MX_E_DEVICE, 0)


def test_wgrad_workspace(lib):
    """The split-contraction workspace is the caller's: its size comes from a host
    query, bad workspace arguments are rejected before any launch."""
    q = lib.mx_grouped_mm_wgrad_workspace_bytes
    # the 576-wide dense wgrad over 16384 tokens: 3 x 16 = 48 tiles of 256x256, so
    # 256 // 48 = 5 splits of fp32 partials, each 576 * 4096 floats
    assert q(1, 16384, 576, 4096, 0) == 5 * 576 * 4096 * 4
    # enough output tiles (8 x 16 x 16 = 2048): no split
    assert q(8, 16384, 4096, 4096, 0) == 0
    # too short a contraction to split (two 256-wide windows per split at least)
    assert q(1, 256, 64, 64, 0) == 0
    # the bf16 operands count 2 bytes per contraction element: more windows, same cap
    assert q(1, 16384, 576, 4096, 1) == 5 * 576 * 4096 * 4
    # a partial's length rounds up to a multiple of 4 floats (16-byte aligned partials)
    assert q(1, 16384, 33, 33, 0) == 16 * ((33 * 33 + 3) // 4 * 4) * 4
    assert q(0, 256, 64, 64, 0) == -1 and q(1, -1, 64, 64, 0) == -1 and q(1, 256, 0, 64, 0) == -1
    w = lib.mx_grouped_mm_wgrad
    assert w(P, P, P, P, None, 1, 256, 64, 64, P2, 0, P2, -16, None) == MX_E_SHAPE  # negative size
    assert w(P, P, P, P, None, 1, 256, 64, 64, P2, 0, P2 + 8, 1024, None) == MX_E_ALIGN  # misaligned
    assert w(P, P, P, P, None, 1, 256, 64, 64, P2, 0, P2, 1024, None) in (MX_E_DEVICE, 0)
    assert w(P, P, P, P, None, 1, 256, 64, 64, P2, 0, None, 0, None) in (MX_E_DEVICE, 0)  # no workspace
    assert lib.mx_grouped_mm_bf16_wgrad(P, P, P2, 3, 104, 36, 64, P2, 0, P2 + 4, 64, None) == MX_E_ALIGN


def test_wgrad_noalloc(lib):
    """The no-allocation wgrad validates like mx_grouped_mm_wgrad; its fixed scratch is
    the largest split any call can make (one round of 256 output tiles of 256 x 256
    fp32 partials): the tightest case fills it exactly."""
    f = lib.mx_grouped_mm_wgrad_noalloc
    assert f(P, P, P, P, None, 1, 40, 64, 64, P2, 0, None) == MX_E_SHAPE  # m % 32
    assert f(P, P, P, P, None, 1, 256, 64, 64, P2, 7, None) == MX_E_DTYPE
    assert f(P, P, P, P, None, 1, 16384, 576, 4096, P2, 1, None) in (MX_E_DEVICE, 0)
    q = lib.mx_grouped_mm_wgrad_workspace_bytes
    assert q(1, 16384, 1024, 4096, 0) == 64 * 1024 * 1024  # 64 tiles, 4 splits of 1024 x 4096 fp32
    for shape in [(1, 16384, 576, 4096), (4, 65536, 576, 4096), (3, 8192, 288, 520), (1, 1 << 22, 32, 64)]:
        assert 0 <= q(*shape, 0) <= 64 * 1024 * 1024


def test_probe_mfma_dot_validation(lib):
    f = lib.mx_probe_mfma_dot
    assert f(0, P, P, P, P, P2, P2, None) in (MX_E_DEVICE, 0)
    assert f(3, P, P, P, P, P2, P2, None) in (MX_E_DEVICE, 0)
    assert f(4, P, P, P, P, P2, P2, None) == MX_E_DTYPE
    assert f(-1, P, P, P, P, P2, P2, None) == MX_E_DTYPE
    assert f(0, None, P, P, P, P2, P2, None) == MX_E_NULL
    assert f(0, P, P, P, P, P2 + 2, P2, None) == MX_E_ALIGN


def test_valid_arguments_without_a_gpu_report_device(lib):
    """With valid arguments and no GPU the library says so instead of launching."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.mx_quantize_dim0(P, 4, 64, 64, P2, P2, None) == MX_E_DEVICE
    assert b"device" in lib.mx_last_error()


def test_python_binding_raises(lib):
    from mxfp8_block_scaled_amd import mx_scale_bytes

    with pytest.raises(ValueError):
        mx_scale_bytes(32, 40)
    assert mx_scale_bytes(64, 512) == 2 * 2 * 256


def test_padded_rows(lib, oracle):
    for rows, G in [(0, 1), (1, 1), (40, 3), (16384, 8), (1000, 1024), (31, 1), (32, 1)]:
        assert lib.mx_padded_rows(rows, G) == oracle.padded_rows(rows, G)
    assert lib.mx_padded_rows(-1, 1) == -1
    assert lib.mx_padded_rows(5, 0) == -1


def test_pad_validation(lib):
    f = lib.mx_pad_token_groups
    assert f(P, 40, 64, 64, P2, 3, P2, 256, P2, None) in (MX_E_DEVICE, 0)  # valid (no GPU here)
    assert f(P, 40, 64, 64, P2, 0, P2, 128, P2, None) == MX_E_SHAPE  # groups
    assert f(P, 40, 64, 64, P2, 1025, P2, 1 << 16, P2, None) == MX_E_SHAPE  # more than 1024 groups
    assert f(P, 40, 64, 64, P2, 3, P2, 224, P2, None) == MX_E_SHAPE  # rows_pad below the bound (256)
    assert b"mx_padded_rows" in lib.mx_last_error()
    assert f(P, 40, 60, 64, P2, 3, P2, 256, P2, None) == MX_E_SHAPE  # cols % 8
    assert f(P, 40, 64, 32, P2, 3, P2, 256, P2, None) == MX_E_LAYOUT  # pitch < cols
    assert f(P, 40, 64, 64, None, 3, P2, 256, P2, None) == MX_E_NULL  # offs
    assert f(P, 40, 64, 64, P2 + 2, 3, P2, 256, P2, None) == MX_E_ALIGN  # offs alignment
    assert f(None, 40, 64, 64, P2, 3, P2, 256, P2, None) == MX_E_NULL  # x
    assert f(P, 40, 64, 64, P2, 3, P2, 256, None, None) == MX_E_NULL  # offs_pad
    assert f(P, (1 << 31) - 16, 64, 64, P2, 3, P2, 1 << 31, P2, None) == MX_E_SHAPE  # int32 offsets overflow
    assert f(None, 0, 64, 64, P2, 2, P2, 256, P2, None) in (MX_E_DEVICE, 0)  # no rows: x may be NULL


def test_unpad_validation(lib):
    f = lib.mx_unpad_token_groups
    assert f(P, 256, 64, 64, P2, 3, P2, 40, 64, 0, None) in (MX_E_DEVICE, 0)
    assert f(P, 256, 64, 64, P2, 3, P2, 40, 64, 2, None) == MX_E_DTYPE
    assert f(P, 256, 6, 6, P2, 3, P2, 40, 6, 0, None) == MX_E_SHAPE  # 24-byte f32 rows
    assert f(P, 256, 4, 4, P2, 3, P2, 40, 4, 1, None) == MX_E_SHAPE  # 8-byte bf16 rows
    assert f(P, 256, 64, 68, P2, 3, P2, 40, 64, 1, None) == MX_E_ALIGN  # bf16 pitch 136 bytes
    assert f(P, 256, 64, 32, P2, 3, P2, 40, 64, 0, None) == MX_E_LAYOUT
    assert f(P, 224, 64, 64, P2, 3, P2, 40, 64, 0, None) == MX_E_SHAPE  # rows_pad too small
    assert f(P, 256, 64, 64, P2, 3, None, 40, 64, 0, None) == MX_E_NULL  # y


def test_backward_arm_calls_validation(lib):
    dq = lib.mx_dequantize
    assert dq(P, P2, 1, 64, 64, 0, P2, None) in (MX_E_DEVICE, 0)
    assert dq(P, P2, 1, 64, 48, 0, P2, None) == MX_E_SHAPE  # cols % 32
    assert dq(P, P2, 1, 36, 64, 1, P2, None) == MX_E_SHAPE  # transposed rows % 8
    assert dq(P, P2, 1, 64, 64, 2, P2, None) == MX_E_DTYPE
    assert dq(P, None, 1, 64, 64, 0, P2, None) == MX_E_NULL
    assert lib.mx_scales_to_logical(P, 64, 40, P2, None) == MX_E_SHAPE
    tr = lib.mx_transpose_bf16
    assert tr(P, 1, 64, 64, 64, P2, None) in (MX_E_DEVICE, 0)
    assert tr(P, 1, 60, 64, 64, P2, None) == MX_E_SHAPE  # rows % 8
    assert tr(P, 1, 64, 64, 32, P2, None) == MX_E_LAYOUT
    f = lib.mx_grouped_mm_bf16_fwd
    assert f(P, P, P2, 3, 100, 40, 64, P2, 0, None) in (MX_E_DEVICE, 0)  # any group rows, n not % 32
    assert f(P, P, P2, 3, 100, 40, 60, P2, 0, None) == MX_E_SHAPE  # k % 8
    assert f(P, P, None, 3, 100, 40, 64, P2, 0, None) == MX_E_SHAPE  # dense with groups
    assert f(P, P, None, 1, 100, 40, (1 << 21) + 8, P2, 0, None) == MX_E_SHAPE  # contraction limit
    assert f(P, P, P2, 1, 100, 40, 64, P2, 5, None) == MX_E_DTYPE
    assert lib.mx_grouped_mm_bf16_dgrad(P, P, P2, 3, 100, 36, 64, P2, 0, None) == MX_E_SHAPE  # n % 8
    assert lib.mx_grouped_mm_bf16_wgrad(P, P, P2, 3, 100, 36, 64, P2, 0, None, 0, None) == MX_E_SHAPE  # m % 8
    assert lib.mx_grouped_mm_bf16_wgrad(P, P, P2, 3, 104, 36, 64, P2, 0, None, 0, None) in (MX_E_DEVICE, 0)


def test_fused_padding_calls_validation(lib):
    e = lib.mx_pad_quantize_ex
    assert e(P, 40, 64, 64, P2, 3, 256, 4, P2, P2, P2, P2, P2, None) in (MX_E_DEVICE, 0)  # MX_FORM_STREAM_T
    assert e(P, 40, 64, 64, P2, 3, 256, 0, P2, P2, P2, P2, P2, None) in (MX_E_DEVICE, 0)
    assert e(P, 40, 64, 64, P2, 3, 256, 1, P2, P2, P2, P2, P2, None) == MX_E_DTYPE  # not a flag here
    assert e(P, 40, 64, 64, P2, 3, 256, 4 | 8, P2, P2, P2, P2, P2, None) == MX_E_DTYPE
    f = lib.mx_pad_quantize_dim0_dim1
    assert f(P, 40, 64, 64, P2, 3, 256, P2, P2, P2, P2, P2, None) in (MX_E_DEVICE, 0)
    assert f(P, 40, 48, 64, P2, 3, 256, P2, P2, P2, P2, P2, None) == MX_E_SHAPE  # cols % 32
    assert f(P, 40, 64, 64, P2, 3, 224, P2, P2, P2, P2, P2, None) == MX_E_SHAPE  # rows_pad below the bound
    assert f(P, 40, 64, 1 << 25, P2, 3, 256, P2, P2, P2, P2, P2, None) == MX_E_SHAPE  # pitch >= 2^25
    assert f(P, 40, 64, 64, P2, 3, 256, P2, P2, None, P2, P2, None) == MX_E_NULL  # q_t
    assert f(P, 40, 64, 64, P2, 3, 256, P2, P2, P2, P2, None, None) == MX_E_NULL  # offs_pad
    g = lib.mx_grouped_mm_fwd_padded
    assert g(P, P, P, P, P2, P2, 3, 256, 40, 64, 64, P2, 0, None) in (MX_E_DEVICE, 0)
    assert g(P, P, P, P, None, P2, 3, 256, 40, 64, 64, P2, 0, None) == MX_E_NULL  # offs_pad
    assert g(P, P, P, P, P2, None, 3, 256, 40, 64, 64, P2, 0, None) == MX_E_NULL  # offs
    assert g(P, P, P, P, P2, P2, 3, 256, 300, 64, 64, P2, 0, None) == MX_E_SHAPE  # m > m_pad
    assert g(P, P, P, P, P2, P2, 3, 256, 40, 40, 64, P2, 0, None) == MX_E_SHAPE  # grouped n % 32
    d = lib.mx_grouped_mm_dgrad_padded
    assert d(P, P, P, P, P2, P2, 3, 256, 40, 64, 64, P2, 0, None) in (MX_E_DEVICE, 0)
    assert d(P, P, P, P, P2, P2, 3, 256, 40, 48, 64, P2, 0, None) == MX_E_SHAPE  # contraction n % 32


def test_check_offs_validation(lib):
    f = lib.mx_check_offs
    assert f(P, 4, 1024, 32, P2, None) in (MX_E_DEVICE, 0)
    assert f(P, 0, 1024, 32, P2, None) == MX_E_SHAPE  # groups
    assert f(P, 4, -1, 32, P2, None) == MX_E_SHAPE  # m
    assert f(P, 4, (1 << 31) + 1, 32, P2, None) == MX_E_SHAPE  # m above 2^31
    assert f(P, 4, 1024, 0, P2, None) == MX_E_SHAPE  # multiple
    assert f(None, 4, 1024, 32, P2, None) == MX_E_NULL
    assert f(P, 4, 1024, 32, None, None) == MX_E_NULL
    assert f(P + 2, 4, 1024, 32, P2, None) == MX_E_ALIGN
    assert f(P, 4, 1024, 32, P2 + 1, None) == MX_E_ALIGN


def test_probe_mfma_validation(lib):
    f = lib.mx_probe_mfma
    assert f(16, P2, None) in (MX_E_DEVICE, 0)
    assert f(0, P2, None) == MX_E_SHAPE
    assert f(1 << 31, P2, None) == MX_E_SHAPE
    assert f(16, None, None) == MX_E_NULL
    assert f(16, P2 + 2, None) == MX_E_ALIGN
