"""The MXFP8 grouped GEMM from its codes, accumulated on the bf16 MFMA.

The block-scaled MFMA (mx_grouped_mm_fwd / _dgrad / _wgrad) truncates the products
inside every run of eight contraction elements, which leaves its fp32 outputs about
1.45e-5 (relative Frobenius) from the exact product of the dequantized operands.
These functions compute the same product from the same codes and scales on
v_mfma_f32_32x32x16_bf16 instead: each operand is dequantized to bf16 (exact: an
E4M3 value times a power of two fits bf16's 8-bit significand wherever the result
lies in bf16's range) and the library's bf16 grouped GEMM accumulates in fp32, which
lands within ~1e-7 of the exact product. They cost the two dequantizations plus a
bf16 GEMM at half the fp8 MFMA rate. Every step runs in the library's kernels; this
module only orders the calls.

The route is the one of the "dequantized" backward override (ao fork PR 10, "Design
notes": gradients from the dequantized forward operands through bf16 grouped GEMMs),
applied to all three passes; dequantization is the MX definition, element times
2^(scale - 127).

Operands as for the MXFP8 calls: fwd a [m, k] and b [G*n, k] dim0
codes; dgrad dy [m, n] dim0 and w_t [G, k, n] dim1 codes; wgrad dy_t [n, m] and
x_t [k, m] dim1 codes; scales in the library's blocked layout. m, n and k are
multiples of 32 (of the bf16 GEMM's 8 as well).
"""

from . import (MX_OUT_BF16, MX_OUT_F32, mx_dequantize, mx_grouped_mm_bf16_dgrad, mx_grouped_mm_bf16_fwd,
               mx_grouped_mm_bf16_wgrad)


def grouped_mm_fwd(a, a_s, b, b_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """Y [m, n] = deq(a) deq(b_g)^T per row group (as mx_grouped_mm_fwd)."""
    a16 = mx_dequantize(a.view(m, k), a_s)
    b16 = mx_dequantize(b.view(-1, k), b_s)
    return mx_grouped_mm_bf16_fwd(a16, b16, offs, m, n, k, groups=groups, out_dtype=out_dtype, out=out)


def grouped_mm_dgrad(dy, dy_s, w_t, w_t_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_BF16, out=None):
    """dX [m, k] = deq(dy) deq(w_t[g]) per row group (as mx_grouped_mm_dgrad)."""
    dy16 = mx_dequantize(dy.view(m, n), dy_s)
    w16 = mx_dequantize(w_t.view(-1, n), w_t_s).view(-1, k, n)  # the blocked scales of [G*k, n] rows
    return mx_grouped_mm_bf16_dgrad(dy16, w16, offs, m, n, k, groups=groups, out_dtype=out_dtype, out=out)


def grouped_mm_wgrad(dy_t, dy_t_s, x_t, x_t_s, offs, m, n, k, groups=None, out_dtype=MX_OUT_F32, out=None,
                     workspace="auto"):
    """dW [G, n, k]: dW[g] = deq(dy_t)[:, rows_g] deq(x_t)[:, rows_g]^T (as mx_grouped_mm_wgrad)."""
    dy16 = mx_dequantize(dy_t.view(n, m), dy_t_s)
    x16 = mx_dequantize(x_t.view(k, m), x_t_s)
    return mx_grouped_mm_bf16_wgrad(dy16, x16, offs, m, n, k, groups=groups, out_dtype=out_dtype, out=out,
                                    workspace=workspace)
