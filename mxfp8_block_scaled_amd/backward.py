"""Backward of the MXFP8 grouped GEMM Y = X W_g^T with a selectable source for the
gradients (ao fork PR 10, "Design notes"), composed from the library's calls:

  "quantized"       the MXFP8 backward: dgrad from dim0(dY) and dim1(W), wgrad from
                    dim1(dY) and dim1(X) (the default)
  "high_precision"  both gradients from the saved bf16 X and W, bf16 grouped GEMMs
  "dequantized"     both gradients from the forward's dim0 codes of X and W
                    dequantized to bf16, bf16 grouped GEMMs (the gradients of the
                    function the quantized forward computes)
  wgrad_with_hp     with "quantized": dgrad as MXFP8, wgrad from the bf16 X and dY

Shapes: X [M, K], W [G, N, K], dY [M, N]; offs int32[G] group ends (any
non-decreasing ends for the bf16 arms; multiples of 32 for the MXFP8 ones).
M, N and K are multiples of 8 for the bf16 arms (16-byte rows). Every step runs in
the library's kernels; this module only orders the calls.
"""

from . import (MX_OUT_BF16, MX_OUT_F32, mx_dequantize, mx_grouped_mm_bf16_dgrad, mx_grouped_mm_bf16_wgrad,
               mx_grouped_mm_dgrad, mx_grouped_mm_wgrad, mx_quantize_dim0, mx_quantize_dim0_dim1, mx_quantize_dim1,
               mx_transpose_bf16)

ARMS = ("quantized", "high_precision", "dequantized")


def grouped_mm_backward(dy, offs, arm="quantized", *, x=None, w=None, x_q=None, x_s=None, w_q=None, w_s=None,
                        wgrad_with_hp=False, dx_dtype=MX_OUT_BF16, dw_dtype=MX_OUT_F32):
    """Returns (dX [M, K], dW [G, N, K]).

    x, w: the saved bf16 input and weight ("quantized", "high_precision",
    wgrad_with_hp). x_q, x_s, w_q, w_s: the forward's dim0 casts of X [M, K] and of
    W as [G*N, K] ("dequantized").
    """
    if arm is None:
        arm = "quantized"
    if arm not in ARMS:
        raise ValueError(f"backward arm {arm!r} is not one of {ARMS}")
    if wgrad_with_hp and arm != "quantized":
        raise ValueError("wgrad_with_hp only modifies the quantized arm (high_precision covers both gradients)")
    M, N = dy.shape
    G = offs.numel()
    if arm == "dequantized":
        K = x_q.shape[1]
        w_t = mx_dequantize(w_q.view(G, N, K), w_s, transpose=True)  # [G, K, N]
        x_t = mx_dequantize(x_q, x_s, transpose=True)  # [K, M]
    else:
        K = x.shape[1]
    if arm == "quantized":
        dyq, dys, dytq, dyts = mx_quantize_dim0_dim1(dy)
        wtq, wts = mx_quantize_dim1(w)
        dx = mx_grouped_mm_dgrad(dyq, dys, wtq, wts, offs, M, N, K, groups=G, out_dtype=dx_dtype)
        if wgrad_with_hp:
            dw = mx_grouped_mm_bf16_wgrad(mx_transpose_bf16(dy), mx_transpose_bf16(x), offs, M, N, K, groups=G,
                                          out_dtype=dw_dtype)
        else:
            xtq, xts = mx_quantize_dim1(x)
            dw = mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, offs, M, N, K, groups=G, out_dtype=dw_dtype)
        return dx, dw
    if arm == "high_precision":
        w_t = mx_transpose_bf16(w)  # [G, K, N]
        x_t = mx_transpose_bf16(x)  # [K, M]
    dy_t = mx_transpose_bf16(dy)  # [N, M]
    dx = mx_grouped_mm_bf16_dgrad(dy, w_t, offs, M, N, K, groups=G, out_dtype=dx_dtype)
    dw = mx_grouped_mm_bf16_wgrad(dy_t, x_t, offs, M, N, K, groups=G, out_dtype=dw_dtype)
    return dx, dw


def quantize_forward_operands(x, w):
    """The forward's dim0 casts that the dequantized arm saves: (x_q, x_s, w_q, w_s)."""
    G, N, K = w.shape
    x_q, x_s = mx_quantize_dim0(x)
    w_q, w_s = mx_quantize_dim0(w.view(G * N, K))
    return x_q, x_s, w_q, w_s
