"""The MXFP8 grouped GEMM from its codes on the bf16 MFMA (mxfp8_block_scaled_amd.precise):
within the IEEE-fp32 figure of 1e-5 (relative Frobenius) of the oracle's float64
product of the same dequantized operands, where the block-scaled MFMA path sits at
~1.45e-5; every fp32 output within the bf16 instruction's per-element bound, bf16
outputs within one ulp of the correctly rounded value or that bound."""

import numpy as np
import pytest

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import precise, synth

from gemm_check import REL_FRO, check_bf16, check_f32
from gpu_util import dev_bf16, dev_i32, host, require_gpu, say

pytestmark = pytest.mark.gpu

M, N, K, SIZES = 2048, 512, 1024, [512, 0, 768, 768]  # one empty group; ends multiples of 32


@pytest.fixture(scope="module")
def data():
    require_gpu()
    rng = np.random.default_rng(31)
    G = len(SIZES)
    return {
        "x": synth.normal_bf16(rng, (M, K), 1.0),
        "w": synth.normal_bf16(rng, (G, N, K), 0.02),
        "dy": synth.normal_bf16(rng, (M, N), 1e-2),
        "offs": np.cumsum(SIZES).astype(np.int32),
        "G": G,
    }


def run_pass(oracle, d, which):
    G, offs = d["G"], d["offs"]
    doffs = dev_i32(offs)
    x, w, dy = d["x"], d["w"], d["dy"]
    if which == "fwd":
        aq, as_ = mx.mx_quantize_dim0(dev_bf16(x))
        bq, bs = mx.mx_quantize_dim0(dev_bf16(w.reshape(G * N, K)))
        call = lambda prec, dt: (precise.grouped_mm_fwd if prec else mx.mx_grouped_mm_fwd)(  # noqa: E731
            aq, as_, bq, bs, doffs, M, N, K, out_dtype=dt)
        oa, oas = oracle.quantize_dim0(x)
        ob, obs = oracle.quantize_dim0(w.reshape(G * N, K))
        ref = oracle.mx_grouped_mm_fwd(oa, oas, ob, obs, offs, G)
        absp = oracle.grouped_mm(np.abs(oracle.dequantize(oa, oas)), np.abs(oracle.dequantize(ob, obs)), offs, G)
        klen = K
    elif which == "dgrad":
        aq, as_ = mx.mx_quantize_dim0(dev_bf16(dy))
        bq, bs = mx.mx_quantize_dim1(dev_bf16(w))  # [G, K, N]
        call = lambda prec, dt: (precise.grouped_mm_dgrad if prec else mx.mx_grouped_mm_dgrad)(  # noqa: E731
            aq, as_, bq, bs, doffs, M, N, K, out_dtype=dt)
        oa, oas = oracle.quantize_dim0(dy)
        parts = [oracle.quantize_dim1(w[g]) for g in range(G)]
        ob, obs = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
        ref = oracle.mx_grouped_mm_fwd(oa, oas, ob, obs, offs, G)
        absp = oracle.grouped_mm(np.abs(oracle.dequantize(oa, oas)), np.abs(oracle.dequantize(ob, obs)), offs, G)
        klen = N
    else:
        _, _, aq, as_ = mx.mx_quantize_dim0_dim1(dev_bf16(dy))  # dy_t [N, M]
        _, _, bq, bs = mx.mx_quantize_dim0_dim1(dev_bf16(x))  # x_t [K, M]
        call = lambda prec, dt: (precise.grouped_mm_wgrad if prec else mx.mx_grouped_mm_wgrad)(  # noqa: E731
            aq, as_, bq, bs, doffs, M, N, K, out_dtype=dt)
        oa, oas = oracle.quantize_dim1(dy)
        ob, obs = oracle.quantize_dim1(x)
        ref = oracle.mx_grouped_mm_wgrad(oa, oas, ob, obs, offs, G)
        absp = oracle.grouped_mm_wgrad(np.abs(oracle.dequantize(oa, oas)), np.abs(oracle.dequantize(ob, obs)), offs,
                                       G)
        klen = max(SIZES)
    return call, ref, absp, klen


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_precise_meets_fp32_figure(oracle, data, which):
    call, ref, absp, klen = run_pass(oracle, data, which)
    got = host(call(True, mx.MX_OUT_F32))
    fast = host(call(False, mx.MX_OUT_F32))
    err, err_fast = oracle.rel_frobenius(got, ref), oracle.rel_frobenius(fast, ref)
    say(f"[precise {which}] rel. Frobenius: bf16-MFMA path {err:.3e}, block-scaled MFMA path {err_fast:.3e}")
    assert err <= REL_FRO, f"{which}: {err:.3e} above {REL_FRO:g}"
    check_f32(oracle, got, ref, f"precise {which} f32", absp, klen)
    got16 = host(call(True, mx.MX_OUT_BF16))
    check_bf16(oracle, got16, ref, absp, klen, f"precise {which} bf16")
    if which == "wgrad":
        assert not got[1].any(), "the empty group's gradient must be zero"


def test_precise_dense_576_layer(oracle):
    """The dense 576-wide layer (offs=None, 32x32 weight scales; dgrad contracts over 576)."""
    require_gpu()
    rng = np.random.default_rng(33)
    m, n, k = 1024, 576, 1024
    x = synth.normal_bf16(rng, (m, k), 1.0)
    w = synth.normal_bf16(rng, (n, k), 0.02)
    dy = synth.normal_bf16(rng, (m, n), 1e-2)
    xq, xs, xtq, xts = mx.mx_quantize_dim0_dim1(dev_bf16(x))
    wq, wqt, wsr, wsc = mx.mx_quantize_weight_32x32(dev_bf16(w))
    dyq, dys, dytq, dyts = mx.mx_quantize_dim0_dim1(dev_bf16(dy))
    oxq, oxs = oracle.quantize_dim0(x)
    oxt, oxts = oracle.quantize_dim1(x)
    owq, owqt, owsr, owsc = oracle.quantize_weight_32x32(w)
    odq, ods = oracle.quantize_dim0(dy)
    odt, odts = oracle.quantize_dim1(dy)
    cases = {
        "fwd": (lambda: precise.grouped_mm_fwd(xq, xs, wq, wsr, None, m, n, k, out_dtype=mx.MX_OUT_F32),
                oracle.mx_grouped_mm_fwd(oxq, oxs, owq, owsr, None, 1),
                oracle.grouped_mm(np.abs(oracle.dequantize(oxq, oxs)), np.abs(oracle.dequantize(owq, owsr)), None, 1),
                k),
        "dgrad": (lambda: precise.grouped_mm_dgrad(dyq, dys, wqt, wsc, None, m, n, k, out_dtype=mx.MX_OUT_F32),
                  oracle.mx_grouped_mm_fwd(odq, ods, owqt, owsc, None, 1),
                  oracle.grouped_mm(np.abs(oracle.dequantize(odq, ods)), np.abs(oracle.dequantize(owqt, owsc)), None,
                                    1),
                  n),
        "wgrad": (lambda: precise.grouped_mm_wgrad(dytq, dyts, xtq, xts, None, m, n, k, out_dtype=mx.MX_OUT_F32),
                  oracle.mx_grouped_mm_wgrad(odt, odts, oxt, oxts, None, 1),
                  oracle.grouped_mm_wgrad(np.abs(oracle.dequantize(odt, odts)), np.abs(oracle.dequantize(oxt, oxts)),
                                          None, 1),
                  m),
    }
    for name, (call, ref, absp, klen) in cases.items():
        got = host(call())
        err = oracle.rel_frobenius(got, ref)
        say(f"[precise dense576 {name}] rel. Frobenius {err:.3e}")
        assert err <= REL_FRO
        check_f32(oracle, got, ref, f"precise dense576 {name} f32", absp, klen)

