"""GPU parity of the backward override arms and their pieces against the oracle.

Dequantization, the logical scale view and the bf16 transposes are bit-exact. The
bf16 grouped GEMMs are bit-exact where every partial sum is representable (small
dyadic operands), including group edges inside a 16-byte chunk of the
contraction, and otherwise within the bars of gemm_check. The three arms are
compared with the oracle's arms.
"""

import numpy as np
import pytest

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import backward, synth

from gemm_check import check_bf16, check_f32
from gpu_util import dev_bf16, dev_i32, host, require_gpu, say, stress_blocks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def test_dequantize_every_amax(oracle):
    """Every bf16 amax pattern (so every scale byte and code), both orientations."""
    blocks = stress_blocks(3)
    n = (blocks.shape[0] // 64) * 64  # whole rows of 8 blocks, a multiple of 8 rows
    x = blocks[:n].reshape(-1, 256)
    say(f"[dequant] stress {x.shape}")
    q, s = mx.mx_quantize_dim0(dev_bf16(x))
    oq, os_ = oracle.quantize_dim0(x)
    want = oracle.dequantize_to_bf16_bits(oq, os_)
    got = host(mx.mx_dequantize(q, s)).view(np.uint16)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} mismatches, first code {oq[bad][0]:#04x} byte {os_[bad[0][0], bad[1][0] // 32]}"
    got_t = host(mx.mx_dequantize(q, s, transpose=True)).view(np.uint16)
    assert np.array_equal(got_t, want.T)


@pytest.mark.parametrize("batch,rows,cols", [(1, 8, 32), (1, 72, 96), (3, 40, 160), (2, 256, 4096)])
def test_dequantize_transposed_shapes(oracle, batch, rows, cols):
    rng = np.random.default_rng(rows + cols)
    x = synth.normal_bf16(rng, (batch * rows, cols), 1.0)
    say(f"[dequant t] batch={batch} rows={rows} cols={cols}")
    q, s = mx.mx_quantize_dim0(dev_bf16(x))
    want = oracle.dequantize_to_bf16_bits(*oracle.quantize_dim0(x)).reshape(batch, rows, cols)
    got = host(mx.mx_dequantize(q.view(batch, rows, cols), s, transpose=True)).view(np.uint16)
    assert np.array_equal(got, want.transpose(0, 2, 1))


def test_scales_to_logical(oracle):
    rng = np.random.default_rng(5)
    x = synth.normal_bf16(rng, (100, 288), 3.0)
    q, s = mx.mx_quantize_dim0(dev_bf16(x))
    _, os_ = oracle.quantize_dim0(x)
    assert np.array_equal(host(mx.mx_scales_to_logical(s, 100, 288)), os_)


@pytest.mark.parametrize("shape", [(8, 8), (72, 136), (3, 40, 200), (8, 4096, 512)])
def test_transpose_bf16(shape):
    rng = np.random.default_rng(sum(shape))
    x = rng.integers(0, 1 << 16, size=shape, dtype=np.uint64).astype(np.uint16)
    say(f"[transpose] {shape}")
    got = host(mx.mx_transpose_bf16(dev_bf16(x))).view(np.uint16)
    assert np.array_equal(got, np.swapaxes(x, -1, -2))


def dyadic(rng, shape):
    """bf16 values in {0, +-0.5, +-1, +-2}: products and their sums stay exact in fp32."""
    vals = np.array([0x0000, 0x3F00, 0xBF00, 0x3F80, 0xBF80, 0x4000, 0xC000], np.uint16)
    return rng.choice(vals, size=shape)


@pytest.mark.parametrize("m,n,k,sizes", [
    (64, 32, 64, None),
    (203, 96, 136, [13, 0, 77, 113]),  # unaligned row groups
    (512, 304, 264, [256, 0, 256]),
])
def test_bf16_fwd_dgrad_exact(oracle, m, n, k, sizes):
    rng = np.random.default_rng(m * n + k)
    G = 1 if sizes is None else len(sizes)
    offs = None if sizes is None else np.cumsum(sizes).astype(np.int32)
    a, b = dyadic(rng, (m, k)), dyadic(rng, (G * n, k))
    say(f"[bf16 fwd exact] m={m} n={n} k={k} sizes={sizes}")
    doffs = None if offs is None else dev_i32(offs)
    got = host(mx.mx_grouped_mm_bf16_fwd(dev_bf16(a), dev_bf16(b), doffs, m, n, k, groups=G, out_dtype=mx.MX_OUT_F32))
    ref = oracle.grouped_mm(oracle.bf16_to_f64(a), oracle.bf16_to_f64(b), offs, G)
    rows = m if offs is None else int(offs[-1])
    assert np.array_equal(got[:rows], ref[:rows].astype(np.float32))
    # dgrad: the same core with the contraction over n
    w_t = dyadic(rng, (G * k, n))
    dy = dyadic(rng, (m, n))
    got = host(mx.mx_grouped_mm_bf16_dgrad(dev_bf16(dy), dev_bf16(w_t), doffs, m, n, k, groups=G,
                                           out_dtype=mx.MX_OUT_F32))
    ref = oracle.grouped_mm(oracle.bf16_to_f64(dy), oracle.bf16_to_f64(w_t), offs, G)
    assert np.array_equal(got[:rows], ref[:rows].astype(np.float32))


@pytest.mark.parametrize("n,k,m,sizes", [
    (64, 96, 64, None),
    (96, 64, 400, [3, 3, 45, 200, 393]),  # edges inside 16-byte chunks (8 tokens), an empty group, tail tokens
    (128, 160, 1024, [1, 511, 1000, 1023, 1024]),
    (32, 40, 16384, [5000, 11007, 16384]),  # long contraction: split path for the narrow output
])
def test_bf16_wgrad_exact(oracle, n, k, m, sizes):
    rng = np.random.default_rng(n + k + m)
    G = 1 if sizes is None else len(sizes)
    offs = None if sizes is None else np.array(sizes, np.int32)
    dy_t, x_t = dyadic(rng, (n, m)), dyadic(rng, (k, m))
    say(f"[bf16 wgrad exact] n={n} k={k} m={m} offs={sizes}")
    got = host(mx.mx_grouped_mm_bf16_wgrad(dev_bf16(dy_t), dev_bf16(x_t), None if offs is None else dev_i32(offs),
                                           m, n, k, groups=G, out_dtype=mx.MX_OUT_F32))
    ref = oracle.grouped_mm_wgrad(oracle.bf16_to_f64(dy_t), oracle.bf16_to_f64(x_t), offs, G)
    assert np.array_equal(got, ref.astype(np.float32))


def test_bf16_large_tilings_exact(oracle):
    """bf16 grouped GEMMs at sizes that pick the large tilings, on dyadic operands (exact
    sums): M-grouped 32 x 17 tiles over K=1088 (bf16 out: 256x256 one wave per SIMD;
    fp32 out: eight waves), M-grouped over a 576-wide contraction (128x256, two blocks
    per CU), K-grouped 8 x 9 x 9 tiles (eight waves) with token edges inside 16-byte
    chunks. Seeded samples of output rows; bf16 outputs are the rounded exact sums."""
    rng = np.random.default_rng(91)

    def rows_of(upto, count):
        return np.sort(rng.choice(upto, size=count, replace=False))

    for m, n, k, G in ((8192, 4128, 1088, 4), (3104, 2336, 576, 3)):
        sizes = rng.multinomial(m - 37, np.full(G, 1.0 / G))
        sizes[1] = 0
        sizes[0] = m - 37 - sizes[1:].sum()
        offs = np.cumsum(sizes).astype(np.int32)
        a, b = dyadic(rng, (m, k)), dyadic(rng, (G * n, k))
        say(f"[bf16 large exact] fwd m={m} n={n} k={k} offs={offs.tolist()}")
        args = (dev_bf16(a), dev_bf16(b), dev_i32(offs), m, n, k)
        got = host(mx.mx_grouped_mm_bf16_fwd(*args, out_dtype=mx.MX_OUT_F32))
        got16 = host(mx.mx_grouped_mm_bf16_fwd(*args, out_dtype=mx.MX_OUT_BF16))
        rows = rows_of(int(offs[-1]), 256)
        sub = np.searchsorted(rows, offs, side="left").astype(np.int32)
        ref = oracle.grouped_mm(oracle.bf16_to_f64(a[rows]), oracle.bf16_to_f64(b), sub, G)
        assert np.array_equal(got[rows], ref.astype(np.float32))
        assert np.array_equal(got16[rows], oracle.round_to_bf16_bits(ref))
    n, k, m, G = 2080, 2080, 2048, 8
    offs = np.array([216, 579, 579, 1100, 1501, 1671, 1861, 2048], np.int32)  # group 2 empty; most edges off 8
    dy_t, x_t = dyadic(rng, (n, m)), dyadic(rng, (k, m))
    say(f"[bf16 large exact] wgrad n={n} k={k} m={m} offs={offs.tolist()}")
    args = (dev_bf16(dy_t), dev_bf16(x_t), dev_i32(offs), m, n, k)
    got = host(mx.mx_grouped_mm_bf16_wgrad(*args, out_dtype=mx.MX_OUT_F32))
    got16 = host(mx.mx_grouped_mm_bf16_wgrad(*args, out_dtype=mx.MX_OUT_BF16))
    rows = rows_of(n, 128)
    ref = oracle.grouped_mm_wgrad(oracle.bf16_to_f64(dy_t[rows]), oracle.bf16_to_f64(x_t), offs, G)
    assert np.array_equal(got[:, rows], ref.astype(np.float32))
    assert np.array_equal(got16[:, rows], oracle.round_to_bf16_bits(ref))
    assert not got[2].any(), "the empty group's gradient must be zero"


@pytest.mark.parametrize("m,n,k,G", [(1000, 256, 512, 4), (2048, 384, 1024, 8)])
def test_bf16_gemm_random(oracle, m, n, k, G):
    rng = np.random.default_rng(m + G)
    sizes = rng.multinomial(m, np.full(G, 1.0 / G))
    offs = np.cumsum(sizes).astype(np.int32)
    a = synth.normal_bf16(rng, (m, k), 1.0)
    b = synth.normal_bf16(rng, (G * n, k), 0.02)
    say(f"[bf16 random] m={m} n={n} k={k} offs={offs.tolist()}")
    doffs = dev_i32(offs)
    got = host(mx.mx_grouped_mm_bf16_fwd(dev_bf16(a), dev_bf16(b), doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
    got16 = host(mx.mx_grouped_mm_bf16_fwd(dev_bf16(a), dev_bf16(b), doffs, m, n, k, out_dtype=mx.MX_OUT_BF16))
    fa, fb = oracle.bf16_to_f64(a), oracle.bf16_to_f64(b)
    ref = oracle.grouped_mm(fa, fb, offs, G)
    absp = oracle.grouped_mm(np.abs(fa), np.abs(fb), offs, G)
    check_f32(oracle, got, ref, "bf16 fwd f32", absp, k)
    check_bf16(oracle, got16, ref, absp, k, "bf16 fwd bf16")
    # wgrad on the same groups (contraction over the unaligned token ranges)
    dy = synth.normal_bf16(rng, (m, n), 1e-2)
    dw = host(mx.mx_grouped_mm_bf16_wgrad(dev_bf16(np.ascontiguousarray(dy.T)), dev_bf16(np.ascontiguousarray(a.T)),
                                          doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
    fdy = oracle.bf16_to_f64(dy)
    refw = oracle.grouped_mm_wgrad(fdy.T, fa.T, offs, G)
    absw = oracle.grouped_mm_wgrad(np.abs(fdy).T, np.abs(fa).T, offs, G)
    check_f32(oracle, dw, refw, "bf16 wgrad f32", absw, m)


@pytest.mark.parametrize("arm", ["high_precision", "dequantized", "quantized", "wgrad_with_hp"])
def test_backward_arms(oracle, arm):
    rng = np.random.default_rng(21)
    M, N, K, G = 640, 192, 256, 4
    sizes = [160, 0, 224, 256] if arm in ("quantized", "wgrad_with_hp") else [150, 0, 233, 257]
    offs = np.cumsum(sizes).astype(np.int32)
    x = synth.normal_bf16(rng, (M, K), 1.0)
    w = synth.normal_bf16(rng, (G, N, K), 0.02)
    dy = synth.normal_bf16(rng, (M, N), 1e-2)
    say(f"[backward arm {arm}] M={M} N={N} K={K} offs={offs.tolist()}")
    dx_, dw_ = dev_bf16(x), dev_bf16(w)
    kw = dict(dx_dtype=mx.MX_OUT_F32, dw_dtype=mx.MX_OUT_F32)
    if arm == "dequantized":
        xq, xs, wq, ws = backward.quantize_forward_operands(dx_, dw_)
        dX, dW = backward.grouped_mm_backward(dev_bf16(dy), dev_i32(offs), "dequantized", x_q=xq, x_s=xs, w_q=wq,
                                              w_s=ws, **kw)
        oxq, oxs = oracle.quantize_dim0(x)
        owq, ows = oracle.quantize_dim0(w.reshape(G * N, K))
        rdx, rdw = oracle.backward_dequantized(oxq, oxs, owq, ows, dy, offs, G)
        xa = oracle.bf16_to_f64(oracle.dequantize_to_bf16_bits(oxq, oxs))
        wa = oracle.bf16_to_f64(oracle.dequantize_to_bf16_bits(owq, ows))
    elif arm == "high_precision":
        dX, dW = backward.grouped_mm_backward(dev_bf16(dy), dev_i32(offs), "high_precision", x=dx_, w=dw_, **kw)
        rdx, rdw = oracle.backward_high_precision(x, w.reshape(G * N, K), dy, offs, G)
        xa, wa = oracle.bf16_to_f64(x), oracle.bf16_to_f64(w.reshape(G * N, K))
    else:
        hp = arm == "wgrad_with_hp"
        dX, dW = backward.grouped_mm_backward(dev_bf16(dy), dev_i32(offs), "quantized", x=dx_, w=dw_,
                                              wgrad_with_hp=hp, **kw)
        odyq, odys = oracle.quantize_dim0(dy)
        parts = [oracle.quantize_dim1(w[g]) for g in range(G)]
        owt, owts = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
        rdx = oracle.mx_grouped_mm_fwd(odyq, odys, owt, owts, offs, G)
        absx = oracle.grouped_mm(np.abs(oracle.dequantize(odyq, odys)), np.abs(oracle.dequantize(owt, owts)), offs, G)
        check_f32(oracle, host(dX), rdx, f"{arm} dX", absx, N)
        if hp:
            fdy, fx = oracle.bf16_to_f64(dy), oracle.bf16_to_f64(x)
            rdw = oracle.grouped_mm_wgrad(fdy.T, fx.T, offs, G)
            absw = oracle.grouped_mm_wgrad(np.abs(fdy).T, np.abs(fx).T, offs, G)
        else:
            odyt, odyts = oracle.quantize_dim1(dy)
            oxt, oxts = oracle.quantize_dim1(x)
            rdw = oracle.mx_grouped_mm_wgrad(odyt, odyts, oxt, oxts, offs, G)
            absw = oracle.grouped_mm_wgrad(np.abs(oracle.dequantize(odyt, odyts)),
                                           np.abs(oracle.dequantize(oxt, oxts)), offs, G)
        check_f32(oracle, host(dW), rdw, f"{arm} dW", absw, M)
        return
    fdy = oracle.bf16_to_f64(dy)
    wa_t = np.concatenate([wa[g * N:(g + 1) * N].T for g in range(G)])
    absx = oracle.grouped_mm(np.abs(fdy), np.abs(wa_t), offs, G)
    absw = oracle.grouped_mm_wgrad(np.abs(fdy).T, np.abs(xa).T, offs, G)
    check_f32(oracle, host(dX), rdx, f"{arm} dX", absx, N)
    check_f32(oracle, host(dW), rdw, f"{arm} dW", absw, M)
