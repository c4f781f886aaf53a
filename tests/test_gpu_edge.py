"""Degenerate and extreme cases on the GPU: empty inputs (zero rows, every group
empty), and GEMMs at the contraction-length limits the header states (2^22 for
MXFP8, 2^21 for bf16), each against the oracle."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import synth

from gemm_check import check_f32, check_mx_fwd, check_mx_wgrad
from gpu_util import dev_bf16, dev_i32, dev_u8, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def phys(oracle, logical):
    return dev_u8(oracle.scales_to_physical(logical))


def test_zero_row_casts():
    say("[edge] zero-row casts")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0")
    q, s = mx.mx_quantize_dim0(x)
    assert q.shape == (0, 64) and s.numel() == 0
    q, s, _, _ = mx.mx_quantize_ex(x, forms=mx.MX_FORM_DIM0, scale_mode=mx.MX_SCALE_FLOOR)
    assert q.shape == (0, 64)
    torch.cuda.synchronize()


def test_zero_row_gemms():
    """m == 0: forward and dgrad have nothing to write; wgrad over an empty
    contraction writes zeros into every group's output."""
    G, n, k = 3, 64, 96
    offs = dev_i32(np.zeros(G, np.int32))
    b = torch.zeros((G * n, k), dtype=torch.uint8, device="cuda:0")
    bs = torch.full((mx.mx_scale_bytes(G * n, k),), 127, dtype=torch.uint8, device="cuda:0")
    empty = torch.empty((0, k), dtype=torch.uint8, device="cuda:0")
    es = torch.empty((0,), dtype=torch.uint8, device="cuda:0")
    say("[edge] m == 0 fwd / dgrad / wgrad")
    out = mx.mx_grouped_mm_fwd(empty, es, b, bs, offs, 0, n, k, groups=G)
    assert out.shape == (0, n)
    dw = torch.full((G, n, k), float("nan"), dtype=torch.float32, device="cuda:0")
    mx.mx_grouped_mm_wgrad(torch.empty((n, 0), dtype=torch.uint8, device="cuda:0"), es,
                           torch.empty((k, 0), dtype=torch.uint8, device="cuda:0"), es, offs, 0, n, k, groups=G,
                           out_dtype=mx.MX_OUT_F32, out=dw)
    assert not host(dw).any()
    dwb = torch.full((G, n, k), float("nan"), dtype=torch.float32, device="cuda:0")
    mx.mx_grouped_mm_bf16_wgrad(torch.empty((n, 0), dtype=torch.bfloat16, device="cuda:0"),
                                torch.empty((k, 0), dtype=torch.bfloat16, device="cuda:0"), offs, 0, n, k, groups=G,
                                out_dtype=mx.MX_OUT_F32, out=dwb)
    assert not host(dwb).any()


def test_every_group_empty(oracle):
    """offs all zero with m > 0: the rows belong to no group, so forward leaves
    the output untouched and wgrad gives zeros."""
    rng = np.random.default_rng(2)
    m, n, k, G = 256, 64, 128, 4
    offs = np.zeros(G, np.int32)
    a, a_s = oracle.quantize_dim0(synth.normal_bf16(rng, (m, k), 1.0))
    b, b_s = oracle.quantize_dim0(synth.normal_bf16(rng, (G * n, k), 0.02))
    out = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda:0")
    say("[edge] every group empty")
    mx.mx_grouped_mm_fwd(dev_u8(a), phys(oracle, a_s), dev_u8(b), phys(oracle, b_s), dev_i32(offs), m, n, k,
                         groups=G, out_dtype=mx.MX_OUT_F32, out=out)
    assert np.all(host(out) == 7.0)
    at, ats = oracle.quantize_dim1(synth.normal_bf16(rng, (m, n), 1.0))
    bt, bts = oracle.quantize_dim1(synth.normal_bf16(rng, (m, k), 1.0))
    dw = mx.mx_grouped_mm_wgrad(dev_u8(at), phys(oracle, ats), dev_u8(bt), phys(oracle, bts), dev_i32(offs), m, n,
                                k, groups=G, out_dtype=mx.MX_OUT_F32)
    assert not host(dw).any()


def random_codes(rng, shape):
    """E4M3 codes of moderate magnitude (no NaN), scales near 1."""
    c = rng.integers(0, 0x60, size=shape).astype(np.uint8) | (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)
    return c


def test_fwd_at_contraction_limit(oracle):
    """Dense forward with k = 2^22, the largest contraction the MXFP8 calls take."""
    rng = np.random.default_rng(22)
    m, n, k = 32, 64, 1 << 22
    a = random_codes(rng, (m, k))
    b = random_codes(rng, (n, k))
    a_s = rng.integers(120, 130, size=(m, k // 32)).astype(np.uint8)
    b_s = rng.integers(120, 130, size=(n, k // 32)).astype(np.uint8)
    say(f"[edge] fwd m={m} n={n} k=2^22")
    got = host(mx.mx_grouped_mm_fwd(dev_u8(a), phys(oracle, a_s), dev_u8(b), phys(oracle, b_s), None, m, n, k,
                                    out_dtype=mx.MX_OUT_F32))
    check_mx_fwd(oracle, got, a, a_s, b, b_s, None, 1, "fwd k=2^22", model_rows=[0])


def test_wgrad_at_contraction_limit(oracle):
    """wgrad over 2^22 tokens in two uneven groups (the split-contraction path)."""
    rng = np.random.default_rng(23)
    n, k, m = 32, 64, 1 << 22
    offs = np.array([1_000_000 // 32 * 32, m], np.int32)
    a = random_codes(rng, (n, m))
    b = random_codes(rng, (k, m))
    a_s = rng.integers(120, 130, size=(n, m // 32)).astype(np.uint8)
    b_s = rng.integers(120, 130, size=(k, m // 32)).astype(np.uint8)
    say(f"[edge] wgrad n={n} k={k} m=2^22 offs={offs.tolist()}")
    got = host(mx.mx_grouped_mm_wgrad(dev_u8(a), phys(oracle, a_s), dev_u8(b), phys(oracle, b_s), dev_i32(offs), m,
                                      n, k, out_dtype=mx.MX_OUT_F32))
    check_mx_wgrad(oracle, got, a, a_s, b, b_s, offs, 2, "wgrad m=2^22", model_rows=[0])


def test_bf16_fwd_at_contraction_limit(oracle):
    """bf16 forward with k = 2^21, the bf16 contraction limit."""
    rng = np.random.default_rng(21)
    m, n, k = 32, 32, 1 << 21
    a = synth.normal_bf16(rng, (m, k), 1.0)
    b = synth.normal_bf16(rng, (n, k), 1.0)
    say(f"[edge] bf16 fwd m={m} n={n} k=2^21")
    got = host(mx.mx_grouped_mm_bf16_fwd(dev_bf16(a), dev_bf16(b), None, m, n, k, out_dtype=mx.MX_OUT_F32))
    fa, fb = oracle.bf16_to_f64(a), oracle.bf16_to_f64(b)
    check_f32(oracle, got, fa @ fb.T, "bf16 fwd k=2^21", np.abs(fa) @ np.abs(fb).T, k)


def test_mfma_probe_runs():
    """The measurement loop runs and leaves finite checksums (4 trips: 2^32 flops)."""
    say("[edge] mfma probe")
    sink = mx.mx_probe_mfma(4)
    s = host(sink)
    assert s.shape == (256,) and np.all(np.isfinite(s)) and np.any(s != 0)
