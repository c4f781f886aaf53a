"""MXFP8 training cast and MXFP8 scaled grouped GEMM for AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/mxfp8.h: each function below has the
name of its C entry point, checks nothing the library checks itself, allocates the
outputs with torch on the input's device and calls the library on the current HIP
stream. Every step of the computation runs in the library's HIP kernels.

Tensors: bf16 inputs may be torch.bfloat16 or int16/uint16 bit patterns; E4M3
codes and E8M0 scales are uint8 tensors; scales are in the library's MFMA-blocked
layout (see `mx_scale_bytes`).
"""

import torch

from . import _lib
from ._lib import MX_OUT_BF16, MX_OUT_F32, MXError  # noqa: F401

__all__ = [
    "mx_scale_bytes",
    "mx_quantize_dim0",
    "mx_quantize_dim1",
    "mx_quantize_dim0_dim1",
    "mx_quantize_ex",
    "MX_FORM_DIM0",
    "MX_FORM_DIM1",
    "MX_SCALE_RCEIL",
    "MX_SCALE_FLOOR",
    "mx_quantize_weight_32x32",
    "mx_grouped_mm_fwd",
    "mx_grouped_mm_dgrad",
    "mx_grouped_mm_wgrad",
    "mx_dequantize",
    "mx_scales_to_logical",
    "mx_transpose_bf16",
    "mx_grouped_mm_bf16_fwd",
    "mx_grouped_mm_bf16_dgrad",
    "mx_grouped_mm_bf16_wgrad",
    "mx_padded_rows",
    "mx_pad_token_groups",
    "mx_pad_quantize_dim0_dim1",
    "mx_grouped_mm_fwd_padded",
    "mx_grouped_mm_dgrad_padded",
    "mx_unpad_token_groups",
    "MXError",
    "library_path",
]


def library_path():
    return _lib.LIB_PATH


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _bf16_bits(x):
    if x.dtype == torch.bfloat16:
        return x
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError(f"expected bf16 data (torch.bfloat16 or 16-bit bit patterns), got {x.dtype}")


def mx_scale_bytes(rows, cols):
    """Bytes of the MFMA-blocked scale buffer of a [rows x cols] quantized matrix."""
    n = _lib.load().mx_scale_bytes(int(rows), int(cols))
    if n < 0:
        raise ValueError(f"mx_scale_bytes({rows}, {cols}): cols must be a non-negative multiple of 32")
    return n


def _u8(n, device):
    return torch.empty(int(n), dtype=torch.uint8, device=device)


def _pitch(x):
    """Row pitch of x (elements); an empty tensor's strides are arbitrary, so its
    rows are taken as packed."""
    if x.numel() == 0:
        return x.shape[-1]
    if x.stride(-1) != 1:
        raise ValueError("x must have unit inner stride")
    return x.stride(-2)


def mx_quantize_dim0(x, q=None, scale=None):
    """1x32 rowwise cast of x [rows, cols] (row pitch x.stride(0)) -> (q [rows, cols], scale)."""
    x = _bf16_bits(x)
    if x.dim() != 2:
        raise ValueError("x must be a 2D tensor")
    rows, cols = x.shape
    ld = _pitch(x)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = _u8(mx_scale_bytes(rows, cols), x.device)
    _lib.call("mx_quantize_dim0", _ptr(x), rows, cols, ld, _ptr(q), _ptr(scale), _stream(x))
    return q, scale


def mx_quantize_dim1(x, q_t=None, scale_t=None):
    """32x1 columnwise cast, written transposed.

    x [rows, cols] or [batch, rows, cols] (batches contiguous) -> q_t [.., cols, rows]
    and the scales of the stacked [batch*cols, rows] matrix.
    """
    x = _bf16_bits(x)
    if x.dim() == 2:
        batch, (rows, cols) = 1, x.shape
    elif x.dim() == 3:
        batch, rows, cols = x.shape
        if x.stride(0) != rows * x.stride(1):
            raise ValueError("batches of x must be contiguous with the row pitch")
    else:
        raise ValueError("x must be 2D or 3D")
    if x.stride(-1) != 1:
        raise ValueError("x must have unit inner stride")
    if q_t is None:
        shape = (cols, rows) if x.dim() == 2 else (batch, cols, rows)
        q_t = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scale_t is None:
        scale_t = _u8(mx_scale_bytes(batch * cols, rows), x.device)
    _lib.call("mx_quantize_dim1", _ptr(x), batch, rows, cols, x.stride(-2), _ptr(q_t), _ptr(scale_t), _stream(x))
    return q_t, scale_t


def mx_quantize_dim0_dim1(x, q=None, scale=None, q_t=None, scale_t=None):
    """Both casts in one pass: x [rows, cols] or [batch, rows, cols] (batches contiguous)
    -> (q [batch*rows, cols], scale, q_t [.., cols, rows], scale_t), the same as
    mx_quantize_dim0 of the stacked rows plus mx_quantize_dim1."""
    x = _bf16_bits(x)
    if x.dim() == 2:
        batch, (rows, cols) = 1, x.shape
    elif x.dim() == 3:
        batch, rows, cols = x.shape
        if x.stride(0) != rows * x.stride(1):
            raise ValueError("batches of x must be contiguous with the row pitch")
    else:
        raise ValueError("x must be 2D or 3D")
    if x.stride(-1) != 1:
        raise ValueError("x must have unit inner stride")
    if q is None:
        q = torch.empty((batch * rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = _u8(mx_scale_bytes(batch * rows, cols), x.device)
    if q_t is None:
        shape = (cols, rows) if x.dim() == 2 else (batch, cols, rows)
        q_t = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scale_t is None:
        scale_t = _u8(mx_scale_bytes(batch * cols, rows), x.device)
    _lib.call("mx_quantize_dim0_dim1", _ptr(x), batch, rows, cols, x.stride(-2), _ptr(q), _ptr(scale), _ptr(q_t),
              _ptr(scale_t), _stream(x))
    return q, scale, q_t, scale_t


MX_FORM_DIM0, MX_FORM_DIM1 = 1, 2
MX_SCALE_RCEIL, MX_SCALE_FLOOR = 0, 1


def mx_quantize_ex(x, forms=MX_FORM_DIM0 | MX_FORM_DIM1, scale_mode=MX_SCALE_RCEIL):
    """Cast with a choice of forms (MX_FORM_DIM0, MX_FORM_DIM1 or both) and scale rule.

    x [rows, cols] or [batch, rows, cols] (batches contiguous). Returns (q, scale,
    q_t, scale_t), None for a form not requested; shapes as mx_quantize_dim0_dim1.
    """
    x = _bf16_bits(x)
    if x.dim() == 2:
        batch, (rows, cols) = 1, x.shape
    elif x.dim() == 3:
        batch, rows, cols = x.shape
        if x.stride(0) != rows * x.stride(1):
            raise ValueError("batches of x must be contiguous with the row pitch")
    else:
        raise ValueError("x must be 2D or 3D")
    ld = _pitch(x)
    q = scale = q_t = scale_t = None
    if forms & MX_FORM_DIM0:
        q = torch.empty((batch * rows, cols), dtype=torch.uint8, device=x.device)
        scale = _u8(mx_scale_bytes(batch * rows, cols), x.device)
    if forms & MX_FORM_DIM1:
        q_t = torch.empty((cols, rows) if x.dim() == 2 else (batch, cols, rows), dtype=torch.uint8, device=x.device)
        scale_t = _u8(mx_scale_bytes(batch * cols, rows), x.device)
    _lib.call("mx_quantize_ex", _ptr(x), batch, rows, cols, ld, int(forms), int(scale_mode), _ptr(q),
              _ptr(scale), _ptr(q_t), _ptr(scale_t), _stream(x))
    return q, scale, q_t, scale_t


def mx_quantize_weight_32x32(w, transposed=True):
    """32x32 weight cast of w [n, k] or [batch, n, k] -> (q, q_t, scale_row, scale_col).

    q_t and scale_col are None when transposed=False.
    """
    w = _bf16_bits(w)
    if w.dim() == 2:
        batch, (n, k) = 1, w.shape
    elif w.dim() == 3:
        batch, n, k = w.shape
        if w.stride(0) != n * w.stride(1):
            raise ValueError("batches of w must be contiguous with the row pitch")
    else:
        raise ValueError("w must be 2D or 3D")
    if w.stride(-1) != 1:
        raise ValueError("w must have unit inner stride")
    lead = () if w.dim() == 2 else (batch,)
    q = torch.empty(lead + (n, k), dtype=torch.uint8, device=w.device)
    s_row = _u8(mx_scale_bytes(batch * n, k), w.device)
    q_t = s_col = None
    if transposed:
        q_t = torch.empty(lead + (k, n), dtype=torch.uint8, device=w.device)
        s_col = _u8(mx_scale_bytes(batch * k, n), w.device)
    _lib.call("mx_quantize_weight_32x32", _ptr(w), batch, n, k, w.stride(-2), _ptr(q), _ptr(q_t), _ptr(s_row),
              _ptr(s_col), _stream(w))
    return q, q_t, s_row, s_col


def _out(shape, out_dtype, device, out):
    if out is not None:
        return out
    dt = torch.float32 if out_dtype == MX_OUT_F32 else torch.bfloat16
    return torch.empty(shape, dtype=dt, device=device)


def _groups(offs, groups):
    if offs is None:
        return 1 if groups is None else groups
    if offs.dtype != torch.int32:
        raise TypeError("offs must be int32")
    return offs.numel() if groups is None else groups


def mx_grouped_mm_fwd(a, a_s, b, b_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """out [m, n] = a [m, k] . b_g [n, k]^T per row group (offs None = dense)."""
    G = _groups(offs, groups)
    out = _out((m, n), out_dtype, a.device, out)
    _lib.call("mx_grouped_mm_fwd", _ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(offs), G, m, n, k, _ptr(out),
              out_dtype, _stream(a))
    return out


def mx_grouped_mm_dgrad(dy, dy_s, w_t, w_t_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """dx [m, k] = dy [m, n] . W_g [n, k] per row group, with W_g^T given as w_t [G*k, n]."""
    G = _groups(offs, groups)
    out = _out((m, k), out_dtype, dy.device, out)
    _lib.call("mx_grouped_mm_dgrad", _ptr(dy), _ptr(dy_s), _ptr(w_t), _ptr(w_t_s), _ptr(offs), G, m, n, k, _ptr(out),
              out_dtype, _stream(dy))
    return out


def mx_grouped_mm_wgrad(dy_t, dy_t_s, x_t, x_t_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_F32, out=None):
    """dw [G, n, k]: dw[g] = dy_t[:, rows_g] . x_t[:, rows_g]^T (empty group -> zeros)."""
    G = _groups(offs, groups)
    out = _out((G, n, k), out_dtype, dy_t.device, out)
    _lib.call("mx_grouped_mm_wgrad", _ptr(dy_t), _ptr(dy_t_s), _ptr(x_t), _ptr(x_t_s), _ptr(offs), G, m, n, k,
              _ptr(out), out_dtype, _stream(dy_t))
    return out


MX_OFFS_DECREASING, MX_OFFS_NOT_MULTIPLE, MX_OFFS_OUT_OF_RANGE = 1, 2, 4


def mx_check_offs(offs, m, multiple=32, result=None):
    """Device check of offs (int32[G]) against the grouped calls' preconditions.

    Returns `result`, a device int32[2] written on the current stream: result[0] = OR
    of MX_OFFS_DECREASING / MX_OFFS_NOT_MULTIPLE / MX_OFFS_OUT_OF_RANGE over the
    groups (0 = valid), result[1] = the first offending group or -1. `multiple` is 32
    for the MXFP8 calls, 1 for the bf16 and padding calls."""
    if offs.dtype != torch.int32 or offs.dim() != 1 or not offs.is_contiguous():
        raise ValueError("offs must be a contiguous 1D int32 tensor")
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=offs.device)
    _lib.call("mx_check_offs", _ptr(offs), offs.numel(), m, multiple, _ptr(result), _stream(offs))
    return result


def mx_probe_mfma(iters, sink=None, device="cuda:0"):
    """Register-only loop of the block-scaled MFMA (iters * 2^30 flops), for timing the
    MXFP8 rate the part sustains. Returns `sink` (device float32[256], written)."""
    if sink is None:
        sink = torch.empty(256, dtype=torch.float32, device=device)
    _lib.call("mx_probe_mfma", int(iters), _ptr(sink), _stream(sink))
    return sink


def mx_padded_rows(rows, groups):
    """Rows of the padded buffer for `rows` token rows in `groups` groups."""
    n = _lib.load().mx_padded_rows(int(rows), int(groups))
    if n < 0:
        raise ValueError(f"mx_padded_rows({rows}, {groups}): need rows in [0, 2^31] and groups >= 1")
    return n


def mx_pad_token_groups(x, offs, rows_pad=None, x_pad=None, offs_pad=None):
    """Pads each token group of x [rows, cols] to a multiple of 32 rows.

    Returns (x_pad [rows_pad, cols], offs_pad int32[G]); offs_pad is written on
    the device and is what the grouped GEMM calls take, with m = rows_pad.
    """
    x = _bf16_bits(x)
    if x.dim() != 2 or (x.numel() and x.stride(1) != 1):
        raise ValueError("x must be a 2D tensor with unit inner stride")
    G = _groups(offs, None)
    rows, cols = x.shape
    ld = x.stride(0) if x.numel() else cols  # an empty tensor's strides are arbitrary
    if rows_pad is None:
        rows_pad = mx_padded_rows(rows, G)
    if x_pad is None:
        x_pad = torch.empty((rows_pad, cols), dtype=x.dtype, device=x.device)
    if offs_pad is None:
        offs_pad = torch.empty(G, dtype=torch.int32, device=x.device)
    _lib.call("mx_pad_token_groups", _ptr(x), rows, cols, ld, _ptr(offs), G, _ptr(x_pad), rows_pad,
              _ptr(offs_pad), _stream(x))
    return x_pad, offs_pad


def mx_unpad_token_groups(y_pad, offs, rows, y=None):
    """Gathers the rows of every group of y_pad [rows_pad, cols] (float32 or bf16)
    back to their unpadded positions in y [rows, cols]."""
    if y_pad.dim() != 2 or y_pad.stride(1) != 1:
        raise ValueError("y_pad must be a 2D tensor with unit inner stride")
    if y_pad.dtype == torch.float32:
        dt = MX_OUT_F32
    elif y_pad.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        dt = MX_OUT_BF16
    else:
        raise TypeError(f"y_pad must be float32 or bf16, got {y_pad.dtype}")
    G = _groups(offs, None)
    rows_pad, cols = y_pad.shape
    if y is None:
        y = torch.empty((rows, cols), dtype=y_pad.dtype, device=y_pad.device)
    _lib.call("mx_unpad_token_groups", _ptr(y_pad), rows_pad, cols, y_pad.stride(0), _ptr(offs), G, _ptr(y), rows,
              y.stride(0), dt, _stream(y_pad))
    return y


def mx_dequantize(q, scale, transpose=False, out=None):
    """Codes q [rows, cols] or [batch, rows, cols] (a dim0 cast's output, scales in
    the blocked layout) -> bf16 [rows, cols], or per batch [cols, rows] when
    `transpose`."""
    if q.dim() == 2:
        batch, (rows, cols) = 1, q.shape
    elif q.dim() == 3:
        batch, rows, cols = q.shape
    else:
        raise ValueError("q must be 2D or 3D")
    if out is None:
        shape = (cols, rows) if transpose else (rows, cols)
        out = torch.empty((batch,) + shape if q.dim() == 3 else shape, dtype=torch.bfloat16, device=q.device)
    _lib.call("mx_dequantize", _ptr(q), _ptr(scale), batch, rows, cols, int(bool(transpose)), _ptr(out), _stream(q))
    return out


def mx_scales_to_logical(scale, rows, cols, out=None):
    """Blocked scale bytes -> logical uint8 [rows, cols / 32]."""
    if out is None:
        out = torch.empty((rows, cols // 32), dtype=torch.uint8, device=scale.device)
    _lib.call("mx_scales_to_logical", _ptr(scale), rows, cols, _ptr(out), _stream(scale))
    return out


def mx_transpose_bf16(x, out=None):
    """bf16 [rows, cols] -> [cols, rows]; [batch, rows, cols] -> [batch, cols, rows]."""
    x = _bf16_bits(x)
    if x.dim() == 2:
        batch, (rows, cols) = 1, x.shape
    elif x.dim() == 3:
        batch, rows, cols = x.shape
        if x.stride(0) != rows * x.stride(1):
            raise ValueError("batches of x must be contiguous with the row pitch")
    else:
        raise ValueError("x must be 2D or 3D")
    if x.numel() and x.stride(-1) != 1:
        raise ValueError("x must have unit inner stride")
    if out is None:
        shape = (cols, rows) if x.dim() == 2 else (batch, cols, rows)
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    ld = x.stride(-2) if x.numel() else cols
    _lib.call("mx_transpose_bf16", _ptr(x), batch, rows, cols, ld, _ptr(out), _stream(x))
    return out


def mx_grouped_mm_bf16_fwd(a, b, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """out [m, n] = a [m, k] . b_g [n, k]^T per row group, bf16 operands."""
    G = _groups(offs, groups)
    out = _out((m, n), out_dtype, a.device, out)
    _lib.call("mx_grouped_mm_bf16_fwd", _ptr(a), _ptr(b), _ptr(offs), G, m, n, k, _ptr(out), out_dtype, _stream(a))
    return out


def mx_grouped_mm_bf16_dgrad(dy, w_t, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """dx [m, k] = dy [m, n] . W_g [n, k] per row group, with W_g^T given as w_t [G*k, n]."""
    G = _groups(offs, groups)
    out = _out((m, k), out_dtype, dy.device, out)
    _lib.call("mx_grouped_mm_bf16_dgrad", _ptr(dy), _ptr(w_t), _ptr(offs), G, m, n, k, _ptr(out), out_dtype,
              _stream(dy))
    return out


def mx_grouped_mm_bf16_wgrad(dy_t, x_t, offs, m, n, k, groups=None, out_dtype=MX_OUT_F32, out=None):
    """dw [G, n, k]: dw[g] = dy_t[:, rows_g] . x_t[:, rows_g]^T, bf16 operands."""
    G = _groups(offs, groups)
    out = _out((G, n, k), out_dtype, dy_t.device, out)
    _lib.call("mx_grouped_mm_bf16_wgrad", _ptr(dy_t), _ptr(x_t), _ptr(offs), G, m, n, k, _ptr(out), out_dtype,
              _stream(dy_t))
    return out


def mx_pad_quantize_dim0_dim1(x, offs, rows_pad=None, q=None, scale=None, q_t=None, scale_t=None, offs_pad=None):
    """Token-group padding fused into the one-pass cast: the casts of
    mx_pad_token_groups(x, offs) without writing the padded bf16 rows.
    Returns (q, scale, q_t, scale_t, offs_pad)."""
    x = _bf16_bits(x)
    if x.dim() != 2:
        raise ValueError("x must be a 2D tensor")
    G = _groups(offs, None)
    rows, cols = x.shape
    ld = _pitch(x)
    if rows_pad is None:
        rows_pad = mx_padded_rows(rows, G)
    dev = x.device
    if q is None:
        q = torch.empty((rows_pad, cols), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = _u8(mx_scale_bytes(rows_pad, cols), dev)
    if q_t is None:
        q_t = torch.empty((cols, rows_pad), dtype=torch.uint8, device=dev)
    if scale_t is None:
        scale_t = _u8(mx_scale_bytes(cols, rows_pad), dev)
    if offs_pad is None:
        offs_pad = torch.empty(G, dtype=torch.int32, device=dev)
    _lib.call("mx_pad_quantize_dim0_dim1", _ptr(x), rows, cols, ld, _ptr(offs), G, rows_pad, _ptr(q), _ptr(scale),
              _ptr(q_t), _ptr(scale_t), _ptr(offs_pad), _stream(x))
    return q, scale, q_t, scale_t, offs_pad


def mx_grouped_mm_fwd_padded(a, a_s, b, b_s, offs_pad, offs, m_pad, m, n, k, out_dtype=MX_OUT_BF16, out=None):
    """Forward on padded token rows, output unpadded: out [m, n]."""
    G = _groups(offs, None)
    out = _out((m, n), out_dtype, a.device, out)
    _lib.call("mx_grouped_mm_fwd_padded", _ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(offs_pad), _ptr(offs), G,
              m_pad, m, n, k, _ptr(out), out_dtype, _stream(a))
    return out


def mx_grouped_mm_dgrad_padded(dy, dy_s, w_t, w_t_s, offs_pad, offs, m_pad, m, n, k, out_dtype=MX_OUT_BF16,
                               out=None):
    """dgrad on padded token rows, output unpadded: dx [m, k]."""
    G = _groups(offs, None)
    out = _out((m, k), out_dtype, dy.device, out)
    _lib.call("mx_grouped_mm_dgrad_padded", _ptr(dy), _ptr(dy_s), _ptr(w_t), _ptr(w_t_s), _ptr(offs_pad), _ptr(offs),
              G, m_pad, m, n, k, _ptr(out), out_dtype, _stream(dy))
    return out
