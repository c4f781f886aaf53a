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
    "MX_FORM_STREAM_T",
    "MX_SCALE_RCEIL",
    "MX_SCALE_FLOOR",
    "mx_quantize_weight_32x32",
    "mx_grouped_mm_fwd",
    "mx_grouped_mm_dgrad",
    "mx_grouped_mm_wgrad",
    "mx_grouped_mm_wgrad_workspace_bytes",
    "mx_grouped_mm_wgrad_noalloc",
    "MX_WGRAD_NOALLOC_SCRATCH_BYTES",
    "mx_dequantize",
    "mx_scales_to_logical",
    "mx_transpose_bf16",
    "mx_grouped_mm_bf16_fwd",
    "mx_grouped_mm_bf16_dgrad",
    "mx_grouped_mm_bf16_wgrad",
    "mx_padded_rows",
    "mx_pad_token_groups",
    "mx_pad_quantize_dim0_dim1",
    "mx_pad_quantize_ex",
    "mx_status_string",
    "mx_last_error",
    "mx_grouped_mm_fwd_padded",
    "mx_grouped_mm_dgrad_padded",
    "mx_unpad_token_groups",
    "mx_probe_mfma",
    "mx_probe_mfma_dot",
    "MX_PROBE_32X32X64",
    "MX_PROBE_16X16X128",
    "MX_PROBE_SWAP",
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


def mx_status_string(status):
    """Name of a status code ("MX_OK", "MX_E_SHAPE", ...)."""
    return _lib.load().mx_status_string(int(status)).decode()


def mx_last_error():
    """This thread's message for its last failed call."""
    return _lib.load().mx_last_error().decode()


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


_U8 = (torch.uint8,)
_I32 = (torch.int32,)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_OUT_DTYPES = {MX_OUT_F32: (torch.float32,), MX_OUT_BF16: _BF16}


def _device_of(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} is on {t.device}; the library works on GPU memory")
    return t.device


def _buf(t, name, dtypes, numel, device):
    """Checks a buffer the library reads or writes: a contiguous tensor of one of
    `dtypes` on `device` with at least `numel` elements. The C library cannot see
    buffer sizes, so this is where a short buffer, a host tensor or a wrong output
    type is caught before a kernel would access memory outside it."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected {' or '.join(str(d) for d in dtypes)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}; the call runs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; the call needs {numel}")
    return t


def _out_dtype(out_dtype):
    if out_dtype not in _OUT_DTYPES:
        raise ValueError(f"out_dtype must be MX_OUT_F32 or MX_OUT_BF16, got {out_dtype!r}")
    return out_dtype


def mx_quantize_dim0(x, q=None, scale=None):
    """1x32 rowwise cast of x [rows, cols] (row pitch x.stride(0)) -> (q [rows, cols], scale)."""
    x = _bf16_bits(x)
    if x.dim() != 2:
        raise ValueError("x must be a 2D tensor")
    rows, cols = x.shape
    ld = _pitch(x)
    dev = _device_of(x, "x")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = _u8(mx_scale_bytes(rows, cols), x.device)
    _buf(q, "q", _U8, rows * cols, dev)
    _buf(scale, "scale", _U8, mx_scale_bytes(rows, cols), dev)
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
    dev = _device_of(x, "x")
    if q_t is None:
        shape = (cols, rows) if x.dim() == 2 else (batch, cols, rows)
        q_t = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scale_t is None:
        scale_t = _u8(mx_scale_bytes(batch * cols, rows), x.device)
    _buf(q_t, "q_t", _U8, batch * rows * cols, dev)
    _buf(scale_t, "scale_t", _U8, mx_scale_bytes(batch * cols, rows), dev)
    _lib.call("mx_quantize_dim1", _ptr(x), batch, rows, cols, x.stride(-2), _ptr(q_t), _ptr(scale_t), _stream(x))
    return q_t, scale_t


def mx_quantize_dim0_dim1(x, q=None, scale=None, q_t=None, scale_t=None, stream_t=False):
    """Both casts in one pass: x [rows, cols] or [batch, rows, cols] (batches contiguous)
    -> (q [batch*rows, cols], scale, q_t [.., cols, rows], scale_t), the same as
    mx_quantize_dim0 of the stacked rows plus mx_quantize_dim1. stream_t: write q_t
    with non-temporal stores (MX_FORM_STREAM_T), for a q_t read only after much other
    traffic; the results are the same."""
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
    dev = _device_of(x, "x")
    _buf(q, "q", _U8, batch * rows * cols, dev)
    _buf(scale, "scale", _U8, mx_scale_bytes(batch * rows, cols), dev)
    _buf(q_t, "q_t", _U8, batch * rows * cols, dev)
    _buf(scale_t, "scale_t", _U8, mx_scale_bytes(batch * cols, rows), dev)
    if stream_t:
        _lib.call("mx_quantize_ex", _ptr(x), batch, rows, cols, x.stride(-2),
                  MX_FORM_DIM0 | MX_FORM_DIM1 | MX_FORM_STREAM_T, MX_SCALE_RCEIL, _ptr(q), _ptr(scale), _ptr(q_t),
                  _ptr(scale_t), _stream(x))
    else:
        _lib.call("mx_quantize_dim0_dim1", _ptr(x), batch, rows, cols, x.stride(-2), _ptr(q), _ptr(scale), _ptr(q_t),
                  _ptr(scale_t), _stream(x))
    return q, scale, q_t, scale_t


MX_FORM_DIM0, MX_FORM_DIM1, MX_FORM_STREAM_T = 1, 2, 4
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


def mx_quantize_weight_32x32(w, transposed=True, q=None, q_t=None, scale_row=None, scale_col=None):
    """32x32 weight cast of w [n, k] or [batch, n, k] -> (q, q_t, scale_row, scale_col).

    q_t and scale_col are None when transposed=False. Outputs may be given (fixed
    buffers, e.g. for graph capture)."""
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
    dev = _device_of(w, "w")
    lead = () if w.dim() == 2 else (batch,)
    if q is None:
        q = torch.empty(lead + (n, k), dtype=torch.uint8, device=w.device)
    if scale_row is None:
        scale_row = _u8(mx_scale_bytes(batch * n, k), w.device)
    _buf(q, "q", _U8, batch * n * k, dev)
    _buf(scale_row, "scale_row", _U8, mx_scale_bytes(batch * n, k), dev)
    if transposed:
        if q_t is None:
            q_t = torch.empty(lead + (k, n), dtype=torch.uint8, device=w.device)
        if scale_col is None:
            scale_col = _u8(mx_scale_bytes(batch * k, n), w.device)
        _buf(q_t, "q_t", _U8, batch * n * k, dev)
        _buf(scale_col, "scale_col", _U8, mx_scale_bytes(batch * k, n), dev)
    else:
        q_t = scale_col = None
    _lib.call("mx_quantize_weight_32x32", _ptr(w), batch, n, k, w.stride(-2), _ptr(q), _ptr(q_t), _ptr(scale_row),
              _ptr(scale_col), _stream(w))
    return q, q_t, scale_row, scale_col


def _out(shape, out_dtype, device, out):
    """The output buffer: `out` checked against the shape and out_dtype, or a new one."""
    _out_dtype(out_dtype)
    n = 1
    for d in shape:
        n *= d
    if out is not None:
        return _buf(out, "out", _OUT_DTYPES[out_dtype], n, device)
    dt = torch.float32 if out_dtype == MX_OUT_F32 else torch.bfloat16
    return torch.empty(shape, dtype=dt, device=device)


def _groups(offs, groups, device=None, name="offs"):
    """Group count: offs.numel() unless `groups` is given; offs must hold that many
    int32 ends on the call's device."""
    if offs is None:
        return 1 if groups is None else groups
    if offs.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    G = offs.numel() if groups is None else groups
    if device is not None:
        _buf(offs, name, _I32, G, device)
    return G


def _mx_operand(t, s, rows, cols, name, device):
    """Codes [rows x cols] and their MFMA-blocked scales."""
    _buf(t, name, _U8, rows * cols, device)
    _buf(s, name + "_scale", _U8, mx_scale_bytes(rows, cols) if rows else 0, device)


def mx_grouped_mm_fwd(a, a_s, b, b_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """out [m, n] = a [m, k] . b_g [n, k]^T per row group (offs None = dense)."""
    dev = _device_of(a, "a")
    G = _groups(offs, groups, dev)
    _mx_operand(a, a_s, m, k, "a", dev)
    _mx_operand(b, b_s, G * n, k, "b", dev)
    out = _out((m, n), out_dtype, dev, out)
    _lib.call("mx_grouped_mm_fwd", _ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(offs), G, m, n, k, _ptr(out),
              out_dtype, _stream(a))
    return out


def mx_grouped_mm_dgrad(dy, dy_s, w_t, w_t_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """dx [m, k] = dy [m, n] . W_g [n, k] per row group, with W_g^T given as w_t [G*k, n]."""
    dev = _device_of(dy, "dy")
    G = _groups(offs, groups, dev)
    _mx_operand(dy, dy_s, m, n, "dy", dev)
    _mx_operand(w_t, w_t_s, G * k, n, "w_t", dev)
    out = _out((m, k), out_dtype, dev, out)
    _lib.call("mx_grouped_mm_dgrad", _ptr(dy), _ptr(dy_s), _ptr(w_t), _ptr(w_t_s), _ptr(offs), G, m, n, k, _ptr(out),
              out_dtype, _stream(dy))
    return out


def mx_grouped_mm_wgrad_workspace_bytes(groups, m, n, k, bf16_operands=False):
    """Workspace bytes with which the wgrad splits its contraction (0: no split)."""
    b = _lib.load().mx_grouped_mm_wgrad_workspace_bytes(int(groups), int(m), int(n), int(k), int(bool(bf16_operands)))
    if b < 0:
        raise ValueError(f"wgrad workspace query: arguments outside the call's limits ({groups}, {m}, {n}, {k})")
    return b


def _workspace(workspace, need, device):
    """(pointer, bytes) of the wgrad workspace: `workspace` as given (any dtype; its
    bytes count; None or empty: the contraction runs unsplit), or, when workspace is
    "auto", a new uint8 tensor of `need` bytes from torch's allocator (kept alive
    by the caching allocator's stream semantics until the work has run)."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be a tensor, None or "auto"')
        if need == 0:
            return None, 0, None
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is None:
        return None, 0, None
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the call's device")
    nbytes = workspace.numel() * workspace.element_size()
    return _ptr(workspace) if nbytes else None, nbytes, workspace


def mx_grouped_mm_wgrad(dy_t, dy_t_s, x_t, x_t_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_F32, out=None,
                        workspace="auto"):
    """dw [G, n, k]: dw[g] = dy_t[:, rows_g] . x_t[:, rows_g]^T (empty group -> zeros).

    workspace: "auto" (a torch allocation of mx_grouped_mm_wgrad_workspace_bytes when
    the call splits its contraction), a caller tensor, or None (never split)."""
    dev = _device_of(dy_t, "dy_t")
    G = _groups(offs, groups, dev)
    _mx_operand(dy_t, dy_t_s, n, m, "dy_t", dev)
    _mx_operand(x_t, x_t_s, k, m, "x_t", dev)
    out = _out((G, n, k), out_dtype, dev, out)
    need = mx_grouped_mm_wgrad_workspace_bytes(G, m, n, k) if workspace == "auto" else 0
    ws_ptr, ws_bytes, _keep = _workspace(workspace, need, dev)
    _lib.call("mx_grouped_mm_wgrad", _ptr(dy_t), _ptr(dy_t_s), _ptr(x_t), _ptr(x_t_s), _ptr(offs), G, m, n, k,
              _ptr(out), out_dtype, ws_ptr, ws_bytes, _stream(dy_t))
    return out


MX_WGRAD_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def mx_grouped_mm_wgrad_noalloc(dy_t, dy_t_s, x_t, x_t_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_F32, out=None):
    """mx_grouped_mm_wgrad without a workspace: a split contraction uses the library's
    fixed per-device scratch (MX_WGRAD_NOALLOC_SCRATCH_BYTES); overlapping calls on one
    device race. `out` must be given by callers that cannot allocate."""
    dev = _device_of(dy_t, "dy_t")
    G = _groups(offs, groups, dev)
    _mx_operand(dy_t, dy_t_s, n, m, "dy_t", dev)
    _mx_operand(x_t, x_t_s, k, m, "x_t", dev)
    out = _out((G, n, k), out_dtype, dev, out)
    _lib.call("mx_grouped_mm_wgrad_noalloc", _ptr(dy_t), _ptr(dy_t_s), _ptr(x_t), _ptr(x_t_s), _ptr(offs), G, m, n,
              k, _ptr(out), out_dtype, _stream(dy_t))
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


MX_PROBE_32X32X64, MX_PROBE_16X16X128, MX_PROBE_SWAP = 0, 1, 2


def mx_probe_mfma_dot(form, a, a_scale, b, b_scale, c=None):
    """One block-scaled MFMA on logical operands (a numerics aid): a, b [R, K] uint8 E4M3
    codes and a_scale, b_scale [R, K/32] uint8 E8M0 bytes on the device (R, K = 32, 64
    for MX_PROBE_32X32X64, 16, 128 for MX_PROBE_16X16X128), c [R, R] float32 (zeros if
    None). Returns d [R, R] float32: c + the instruction's dot of row i of a with row j
    of b. form | MX_PROBE_SWAP passes b as the instruction's first operand."""
    R, K = (16, 128) if form & 1 else (32, 64)
    for name, t, shape in (("a", a, (R, K)), ("b", b, (R, K)), ("a_scale", a_scale, (R, K // 32)),
                           ("b_scale", b_scale, (R, K // 32))):
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 device tensor of shape {shape}")
    if c is None:
        c = torch.zeros((R, R), dtype=torch.float32, device=a.device)
    if c.dtype != torch.float32 or tuple(c.shape) != (R, R) or not c.is_cuda or not c.is_contiguous():
        raise ValueError(f"c must be a contiguous float32 device tensor of shape {(R, R)}")
    d = torch.empty_like(c)
    _lib.call("mx_probe_mfma_dot", int(form), _ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), _ptr(c), _ptr(d),
              _stream(a))
    return d


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
    dev = _device_of(x, "x")
    G = _groups(offs, None, dev)
    rows, cols = x.shape
    ld = x.stride(0) if x.numel() else cols  # an empty tensor's strides are arbitrary
    if rows_pad is None:
        rows_pad = mx_padded_rows(rows, G)
    if x_pad is None:
        x_pad = torch.empty((rows_pad, cols), dtype=x.dtype, device=x.device)
    if offs_pad is None:
        offs_pad = torch.empty(G, dtype=torch.int32, device=x.device)
    _buf(x_pad, "x_pad", _BF16, rows_pad * cols, dev)
    _buf(offs_pad, "offs_pad", _I32, G, dev)
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
    dev = _device_of(y_pad, "y_pad")
    G = _groups(offs, None, dev)
    rows_pad, cols = y_pad.shape
    if y is None:
        y = torch.empty((rows, cols), dtype=y_pad.dtype, device=y_pad.device)
    if y.dtype != y_pad.dtype or y.device != dev or y.dim() != 2 or y.shape[1] != cols or y.shape[0] < rows or \
            (y.numel() and y.stride(1) != 1):
        raise ValueError("y must be a 2D tensor of y_pad's dtype and device, unit inner stride, [>= rows, cols]")
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
    dev = _device_of(a, "a")
    G = _groups(offs, groups, dev)
    _buf(a, "a", _BF16, m * k, dev)
    _buf(b, "b", _BF16, G * n * k, dev)
    out = _out((m, n), out_dtype, dev, out)
    _lib.call("mx_grouped_mm_bf16_fwd", _ptr(a), _ptr(b), _ptr(offs), G, m, n, k, _ptr(out), out_dtype, _stream(a))
    return out


def mx_grouped_mm_bf16_dgrad(dy, w_t, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """dx [m, k] = dy [m, n] . W_g [n, k] per row group, with W_g^T given as w_t [G*k, n]."""
    dev = _device_of(dy, "dy")
    G = _groups(offs, groups, dev)
    _buf(dy, "dy", _BF16, m * n, dev)
    _buf(w_t, "w_t", _BF16, G * k * n, dev)
    out = _out((m, k), out_dtype, dev, out)
    _lib.call("mx_grouped_mm_bf16_dgrad", _ptr(dy), _ptr(w_t), _ptr(offs), G, m, n, k, _ptr(out), out_dtype,
              _stream(dy))
    return out


def mx_grouped_mm_bf16_wgrad(dy_t, x_t, offs, m, n, k, groups=None, out_dtype=MX_OUT_F32, out=None,
                             workspace="auto"):
    """dw [G, n, k]: dw[g] = dy_t[:, rows_g] . x_t[:, rows_g]^T, bf16 operands;
    workspace as for mx_grouped_mm_wgrad."""
    dev = _device_of(dy_t, "dy_t")
    G = _groups(offs, groups, dev)
    _buf(dy_t, "dy_t", _BF16, n * m, dev)
    _buf(x_t, "x_t", _BF16, k * m, dev)
    out = _out((G, n, k), out_dtype, dev, out)
    need = mx_grouped_mm_wgrad_workspace_bytes(G, m, n, k, True) if workspace == "auto" else 0
    ws_ptr, ws_bytes, _keep = _workspace(workspace, need, dev)
    _lib.call("mx_grouped_mm_bf16_wgrad", _ptr(dy_t), _ptr(x_t), _ptr(offs), G, m, n, k, _ptr(out), out_dtype,
              ws_ptr, ws_bytes, _stream(dy_t))
    return out


def mx_pad_quantize_dim0_dim1(x, offs, rows_pad=None, q=None, scale=None, q_t=None, scale_t=None, offs_pad=None,
                              stream_t=False):
    """Token-group padding fused into the one-pass cast: the casts of
    mx_pad_token_groups(x, offs) without writing the padded bf16 rows.
    Returns (q, scale, q_t, scale_t, offs_pad). stream_t: q_t written with
    non-temporal stores (MX_FORM_STREAM_T), the same values."""
    x = _bf16_bits(x)
    if x.dim() != 2:
        raise ValueError("x must be a 2D tensor")
    dev = _device_of(x, "x")
    G = _groups(offs, None, dev)
    rows, cols = x.shape
    ld = _pitch(x)
    if rows_pad is None:
        rows_pad = mx_padded_rows(rows, G)
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
    _buf(q, "q", _U8, rows_pad * cols, dev)
    _buf(scale, "scale", _U8, mx_scale_bytes(rows_pad, cols), dev)
    _buf(q_t, "q_t", _U8, rows_pad * cols, dev)
    _buf(scale_t, "scale_t", _U8, mx_scale_bytes(cols, rows_pad), dev)
    _buf(offs_pad, "offs_pad", _I32, G, dev)
    _lib.call("mx_pad_quantize_ex", _ptr(x), rows, cols, ld, _ptr(offs), G, rows_pad,
              MX_FORM_STREAM_T if stream_t else 0, _ptr(q), _ptr(scale), _ptr(q_t), _ptr(scale_t), _ptr(offs_pad),
              _stream(x))
    return q, scale, q_t, scale_t, offs_pad


def mx_pad_quantize_ex(x, offs, flags=0, rows_pad=None, q=None, scale=None, q_t=None, scale_t=None, offs_pad=None):
    """mx_pad_quantize_dim0_dim1 with the C call's flags: 0 or MX_FORM_STREAM_T."""
    if flags not in (0, MX_FORM_STREAM_T):
        raise ValueError(f"flags = {flags} must be 0 or MX_FORM_STREAM_T")
    return mx_pad_quantize_dim0_dim1(x, offs, rows_pad, q, scale, q_t, scale_t, offs_pad,
                                     stream_t=flags == MX_FORM_STREAM_T)


def mx_grouped_mm_fwd_padded(a, a_s, b, b_s, offs_pad, offs, m_pad, m, n, k, out_dtype=MX_OUT_BF16, out=None):
    """Forward on padded token rows, output unpadded: out [m, n]."""
    dev = _device_of(a, "a")
    G = _groups(offs, None, dev)
    _groups(offs_pad, G, dev, "offs_pad")
    _mx_operand(a, a_s, m_pad, k, "a", dev)
    _mx_operand(b, b_s, G * n, k, "b", dev)
    out = _out((m, n), out_dtype, dev, out)
    _lib.call("mx_grouped_mm_fwd_padded", _ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(offs_pad), _ptr(offs), G,
              m_pad, m, n, k, _ptr(out), out_dtype, _stream(a))
    return out


def mx_grouped_mm_dgrad_padded(dy, dy_s, w_t, w_t_s, offs_pad, offs, m_pad, m, n, k, out_dtype=MX_OUT_BF16,
                               out=None):
    """dgrad on padded token rows, output unpadded: dx [m, k]."""
    dev = _device_of(dy, "dy")
    G = _groups(offs, None, dev)
    _groups(offs_pad, G, dev, "offs_pad")
    _mx_operand(dy, dy_s, m_pad, n, "dy", dev)
    _mx_operand(w_t, w_t_s, G * k, n, "w_t", dev)
    out = _out((m, k), out_dtype, dev, out)
    _lib.call("mx_grouped_mm_dgrad_padded", _ptr(dy), _ptr(dy_s), _ptr(w_t), _ptr(w_t_s), _ptr(offs_pad), _ptr(offs),
              G, m_pad, m, n, k, _ptr(out), out_dtype, _stream(dy))
    return out
