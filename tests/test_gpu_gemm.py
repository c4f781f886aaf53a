"""GPU parity of the MXFP8 grouped GEMM (forward, dgrad, wgrad) against the oracle.

Bit-exact fp32 output where every partial sum is exactly representable (codes in
{0, +-0.5, +-1, +-2}, scales 2^-1..2^1); otherwise the bars of gemm_check: every
output within the tolerance of the block-scaled MFMA's arithmetic model
(tests/mfma_model.py) and within the model's worst-case bound of the exact value;
relative Frobenius error and bf16 ulp counts reported.
"""

import numpy as np
import pytest

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import synth

from gemm_check import check_mx_fwd, check_mx_wgrad
from gpu_util import dev_bf16, dev_i32, dev_u8, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def phys(oracle, logical):
    return dev_u8(oracle.scales_to_physical(logical))


def exact_operands(rng, rows, k):
    choices = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], np.uint8)
    q = rng.choice(choices, size=(rows, k))
    s = rng.integers(126, 129, size=(rows, k // 32)).astype(np.uint8)
    return q, s


@pytest.mark.parametrize("m,n,k,sizes", [
    (256, 128, 256, None),
    (100, 96, 576, None),
    (352, 64, 512, [32, 0, 96, 224]),
    (640, 160, 1024, [0, 256, 0, 128, 256]),
])
def test_fwd_exact_integer(oracle, m, n, k, sizes):
    rng = np.random.default_rng(m + n + k)
    G = 1 if sizes is None else len(sizes)
    a_q, a_s = exact_operands(rng, m, k)
    b_q, b_s = exact_operands(rng, G * n, k)
    offs = None if sizes is None else np.cumsum(sizes).astype(np.int32)
    say(f"[gemm fwd exact] m={m} n={n} k={k} sizes={sizes}")
    out = mx.mx_grouped_mm_fwd(dev_u8(a_q), phys(oracle, a_s), dev_u8(b_q), phys(oracle, b_s),
                               None if offs is None else dev_i32(offs), m, n, k, groups=G, out_dtype=mx.MX_OUT_F32)
    ref = oracle.mx_grouped_mm_fwd(a_q, a_s, b_q, b_s, offs, G)
    got = host(out)
    assert np.array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("n,k,m,sizes", [
    (64, 96, 288, [32, 32, 96, 224, 288]),
    (100, 64, 256, None),
    (128, 160, 608, [0, 64, 96, 96, 480, 608]),
])
def test_wgrad_exact_integer(oracle, n, k, m, sizes):
    """Group boundaries at odd 32-blocks, empty groups, ragged n and k."""
    rng = np.random.default_rng(n * k + m)
    offs = None if sizes is None else np.array(sizes, np.int32)
    G = 1 if sizes is None else len(sizes)
    dy_t, dy_s = exact_operands(rng, n, m)
    x_t, x_s = exact_operands(rng, k, m)
    say(f"[gemm wgrad exact] n={n} k={k} m={m} offs={sizes}")
    out = mx.mx_grouped_mm_wgrad(dev_u8(dy_t), phys(oracle, dy_s), dev_u8(x_t), phys(oracle, x_s),
                                 None if offs is None else dev_i32(offs), m, n, k, groups=G, out_dtype=mx.MX_OUT_F32)
    ref = oracle.mx_grouped_mm_wgrad(dy_t, dy_s, x_t, x_s, offs, G)
    got = host(out)
    assert np.array_equal(got, ref.astype(np.float32))
    if offs is not None:
        starts = np.concatenate([[0], offs[:-1]])
        for g in range(G):
            if starts[g] == offs[g]:
                assert np.all(got[g] == 0)


@pytest.mark.parametrize("G,seed,nw", [(96, 1, 288), (300, 2, 288), (2000, 3, 64)])
def test_many_groups_exact(oracle, G, seed, nw):
    """Many small groups, about a third of them empty: the forward's group search (64
    groups per wave-scan step, so 2, 5 and 32 steps here) and the wgrad's slice-major
    order over G groups (each group's raster in several slices of uneven length),
    full outputs bit-exact."""
    rng = np.random.default_rng(1000 + seed)
    units = rng.integers(0, 4, size=G) * (rng.random(G) > 0.35)
    sizes = 32 * units
    offs = np.cumsum(sizes).astype(np.int32)
    m = int(offs[-1]) + 64  # rows past the last group: unwritten (fwd), unread (wgrad)
    n, k = 96, 160
    a_q, a_s = exact_operands(rng, m, k)
    b_q, b_s = exact_operands(rng, G * n, k)
    say(f"[gemm many groups] fwd G={G} m={m} n={n} k={k}")
    got = host(mx.mx_grouped_mm_fwd(dev_u8(a_q), phys(oracle, a_s), dev_u8(b_q), phys(oracle, b_s), dev_i32(offs),
                                    m, n, k, groups=G, out_dtype=mx.MX_OUT_F32))
    ref = oracle.mx_grouped_mm_fwd(a_q, a_s, b_q, b_s, offs, G)
    rows = int(offs[-1])
    assert np.array_equal(got[:rows], ref[:rows].astype(np.float32))
    # wgrad: dW_g = dY_g^T X_g over each group's token range; [G, nw, 96] outputs
    kw = 96
    dy_t, dy_s = exact_operands(rng, nw, m)
    x_t, x_s = exact_operands(rng, kw, m)
    say(f"[gemm many groups] wgrad G={G} n={nw} k={kw} m={m}")
    got = host(mx.mx_grouped_mm_wgrad(dev_u8(dy_t), phys(oracle, dy_s), dev_u8(x_t), phys(oracle, x_s), dev_i32(offs),
                                      m, nw, kw, groups=G, out_dtype=mx.MX_OUT_F32))
    ref = oracle.mx_grouped_mm_wgrad(dy_t, dy_s, x_t, x_s, offs, G)
    assert np.array_equal(got, ref.astype(np.float32))
    assert not got[sizes == 0].any()


def test_dgrad_exact_integer(oracle):
    rng = np.random.default_rng(3)
    m, n, k, sizes = 320, 96, 128, [64, 0, 256]
    G = len(sizes)
    offs = np.cumsum(sizes).astype(np.int32)
    dy, dy_s = exact_operands(rng, m, n)
    w_t, w_t_s = exact_operands(rng, G * k, n)
    say("[gemm dgrad exact]")
    out = mx.mx_grouped_mm_dgrad(dev_u8(dy), phys(oracle, dy_s), dev_u8(w_t), phys(oracle, w_t_s), dev_i32(offs),
                                 m, n, k, groups=G, out_dtype=mx.MX_OUT_F32)
    ref = oracle.mx_grouped_mm_fwd(dy, dy_s, w_t, w_t_s, offs, G)
    assert np.array_equal(host(out), ref.astype(np.float32))


def test_small_linear_forward(oracle):
    """256^3 dense MXFP8 linear with zero and outlier blocks, fp32 out (GPU casts feed the GEMM)."""
    d = synth.linear_small(0)
    say("[gemm] small linear fwd")
    a_q, a_s = mx.mx_quantize_dim0(dev_bf16(d["a"]))
    b_q, b_s = mx.mx_quantize_dim0(dev_bf16(d["b"]))
    y = host(mx.mx_grouped_mm_fwd(a_q, a_s, b_q, b_s, None, 256, 256, 256, out_dtype=mx.MX_OUT_F32))
    oa, oas = oracle.quantize_dim0(d["a"])
    ob, obs = oracle.quantize_dim0(d["b"])
    ref = oracle.mx_grouped_mm_fwd(oa, oas, ob, obs, None, 1)
    check_mx_fwd(oracle, y, oa, oas, ob, obs, None, 1, "fwd 256^3")
    unq = oracle.bf16_to_f64(d["a"]) @ oracle.bf16_to_f64(d["b"]).T
    sq = oracle.sqnr_db(y, unq)
    say(f"    SQNR vs unquantized: {sq:.2f} dB")
    assert sq >= 25.0


def grouped_case(seed, m, n, k, G, std_b=0.02):
    rng = np.random.default_rng(seed)
    sizes = synth.multinomial_groups(rng, m, G)
    sizes[0] = 0 if G > 2 else sizes[0]
    sizes[-1] += m - sizes.sum()
    return (synth.offs_from_sizes(sizes), synth.normal_bf16(rng, (m, k), 1.0),
            synth.normal_bf16(rng, (G, n, k), std_b), synth.normal_bf16(rng, (m, n), 1e-2))


@pytest.mark.parametrize("m,n,k,G", [(512, 256, 512, 4), (1024, 384, 576, 3), (768, 128, 1024, 1)])
def test_grouped_fwd_dgrad_wgrad(oracle, m, n, k, G):
    offs, x, w, dy = grouped_case(m + n + k, m, n, k, G)
    say(f"[gemm grouped] m={m} n={n} k={k} G={G} offs={offs.tolist()}")
    doffs = dev_i32(offs)
    xq, xs = mx.mx_quantize_dim0(dev_bf16(x))
    wq, ws = mx.mx_quantize_dim0(dev_bf16(w.reshape(G * n, k)))
    y32 = host(mx.mx_grouped_mm_fwd(xq, xs, wq, ws, doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
    y16 = host(mx.mx_grouped_mm_fwd(xq, xs, wq, ws, doffs, m, n, k, out_dtype=mx.MX_OUT_BF16))
    oxq, oxs = oracle.quantize_dim0(x)
    owq, ows = oracle.quantize_dim0(w.reshape(G * n, k))
    check_mx_fwd(oracle, y32, oxq, oxs, owq, ows, offs, G, "fwd f32")
    check_mx_fwd(oracle, y16, oxq, oxs, owq, ows, offs, G, "fwd bf16", out_bf16=True)

    # dgrad: dX = dY . W_g, with W_g^T from the dim1 cast of the [G, n, k] weight
    dyq, dys = mx.mx_quantize_dim0(dev_bf16(dy))
    wtq, wts = mx.mx_quantize_dim1(dev_bf16(w))
    dx = host(mx.mx_grouped_mm_dgrad(dyq, dys, wtq, wts, doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
    odyq, odys = oracle.quantize_dim0(dy)
    parts = [oracle.quantize_dim1(w[g]) for g in range(G)]
    owt = np.concatenate([p[0] for p in parts])
    owts = np.concatenate([p[1] for p in parts])
    check_mx_fwd(oracle, dx, odyq, odys, owt, owts, offs, G, "dgrad f32")

    # wgrad: dW_g = dY_g^T . X_g from dim1 casts
    dytq, dyts = mx.mx_quantize_dim1(dev_bf16(dy))
    xtq, xts = mx.mx_quantize_dim1(dev_bf16(x))
    dw = host(mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
    odyt, odyts = oracle.quantize_dim1(dy)
    oxt, oxts = oracle.quantize_dim1(x)
    check_mx_wgrad(oracle, dw, odyt, odyts, oxt, oxts, offs, G, "wgrad f32")


def test_dense_linear_4096(oracle):
    """MXFP8Linear fwd+bwd at M=N=4096, K=2048 with 32x32 weight scales."""
    d = synth.linear_4096(0)
    x, w, dy = d["x"], d["w"], d["dy"]
    M, K = x.shape
    N = w.shape[0]
    say("[gemm dense 4096] casts")
    xq, xs = mx.mx_quantize_dim0(dev_bf16(x))
    wq, wqt, wsr, wsc = mx.mx_quantize_weight_32x32(dev_bf16(w))
    dyq, dys = mx.mx_quantize_dim0(dev_bf16(dy))
    dytq, dyts = mx.mx_quantize_dim1(dev_bf16(dy))
    xtq, xts = mx.mx_quantize_dim1(dev_bf16(x))
    say("[gemm dense 4096] fwd/dgrad/wgrad")
    y = host(mx.mx_grouped_mm_fwd(xq, xs, wq, wsr, None, M, N, K, out_dtype=mx.MX_OUT_F32))
    dx = host(mx.mx_grouped_mm_dgrad(dyq, dys, wqt, wsc, None, M, N, K, out_dtype=mx.MX_OUT_F32))
    dw = host(mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, None, M, N, K, out_dtype=mx.MX_OUT_F32))
    oxq, oxs = oracle.quantize_dim0(x)
    owq, owqt, owsr, owsc = oracle.quantize_weight_32x32(w)
    rows = np.sort(np.random.default_rng(0).choice(M, 256, replace=False))
    mrows = np.arange(8)  # the model on 8 of the sampled rows (8 x 4096 x 2048 products each)
    check_mx_fwd(oracle, y[rows], oxq[rows], oxs[rows], owq, owsr, None, 1, "fwd", model_rows=mrows)
    odyq, odys = oracle.quantize_dim0(dy)
    check_mx_fwd(oracle, dx[rows], odyq[rows], odys[rows], owqt, owsc, None, 1, "dgrad", model_rows=mrows)
    odyt, odyts = oracle.quantize_dim1(dy)
    oxt, oxts = oracle.quantize_dim1(x)
    check_mx_fwd(oracle, dw[0][rows], odyt[rows], odyts[rows], oxt, oxts, None, 1, "wgrad", model_rows=mrows)


def test_gemm_deterministic():
    offs, x, w, _ = grouped_case(5, 512, 256, 512, 4)
    xq, xs = mx.mx_quantize_dim0(dev_bf16(x))
    wq, ws = mx.mx_quantize_dim0(dev_bf16(w.reshape(-1, 512)))
    doffs = dev_i32(offs)
    a = host(mx.mx_grouped_mm_fwd(xq, xs, wq, ws, doffs, 512, 256, 512, out_dtype=mx.MX_OUT_F32))
    b = host(mx.mx_grouped_mm_fwd(xq, xs, wq, ws, doffs, 512, 256, 512, out_dtype=mx.MX_OUT_F32))
    assert np.array_equal(a, b)


def test_fwd_two_rounds_ragged_groups(oracle):
    """M=8192, N=4096 in 4 ragged groups (every group ends mid-tile), full output compared."""
    m, n, k, G = 8192, 4096, 256, 4
    rng = np.random.default_rng(21)
    sizes = np.array([2080, 1984, 2112, 2016])  # ragged: every group ends mid-tile
    offs = synth.offs_from_sizes(sizes)
    x = synth.normal_bf16(rng, (m, k), 1.0)
    w = synth.normal_bf16(rng, (G, n, k), 0.02)
    say(f"[gemm 2-round fwd] offs={offs.tolist()}")
    xq, xs = mx.mx_quantize_dim0(dev_bf16(x))
    wq, ws = mx.mx_quantize_dim0(dev_bf16(w.reshape(G * n, k)))
    y = host(mx.mx_grouped_mm_fwd(xq, xs, wq, ws, dev_i32(offs), m, n, k, out_dtype=mx.MX_OUT_F32))
    oxq, oxs = oracle.quantize_dim0(x)
    owq, ows = oracle.quantize_dim0(w.reshape(G * n, k))
    edges = np.concatenate([[0], offs[:-1], offs - 1])
    model_rows = np.unique(np.concatenate([edges, np.random.default_rng(3).integers(0, m, 48)]))
    check_mx_fwd(oracle, y, oxq, oxs, owq, ows, offs, G, "2-round fwd f32", model_rows=model_rows)


def test_wgrad_ragged_tile_grid(oracle):
    """K-grouped, G=4 (one empty), 2560 x 3328 outputs: partial tiles on both output edges."""
    m, n, k, G = 256, 2560, 3328, 4
    rng = np.random.default_rng(22)
    offs = synth.offs_from_sizes(np.array([96, 0, 64, 96]))
    dy = synth.normal_bf16(rng, (m, n), 1e-2)
    x = synth.normal_bf16(rng, (m, k), 1.0)
    say(f"[gemm ragged wgrad] offs={offs.tolist()}")
    dytq, dyts = mx.mx_quantize_dim1(dev_bf16(dy))
    xtq, xts = mx.mx_quantize_dim1(dev_bf16(x))
    dw = host(mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, dev_i32(offs), m, n, k, out_dtype=mx.MX_OUT_F32))
    odyt, odyts = oracle.quantize_dim1(dy)
    oxt, oxts = oracle.quantize_dim1(x)
    check_mx_wgrad(oracle, dw, odyt, odyts, oxt, oxts, offs, G, "ragged wgrad f32")


@pytest.mark.parametrize("out_dtype", [mx.MX_OUT_F32, mx.MX_OUT_BF16])
def test_wgrad_split_contraction(oracle, out_dtype):
    """576 x 512 outputs per group over 8192 tokens: few output tiles, so the contraction
    is split (fp32 partials summed in order); group 0 ends off a 256 boundary, group 1 is empty."""
    m, n, k = 8192, 576, 512
    sizes = np.array([2080, 0, 6112])
    G = len(sizes)
    offs = synth.offs_from_sizes(sizes)
    rng = np.random.default_rng(23)
    dy = synth.normal_bf16(rng, (m, n), 1e-2)
    x = synth.normal_bf16(rng, (m, k), 1.0)
    say(f"[gemm split wgrad] offs={offs.tolist()} out={'bf16' if out_dtype else 'f32'}")
    dytq, dyts = mx.mx_quantize_dim1(dev_bf16(dy))
    xtq, xts = mx.mx_quantize_dim1(dev_bf16(x))
    dw = mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, dev_i32(offs), m, n, k, out_dtype=out_dtype)
    again = mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, dev_i32(offs), m, n, k, out_dtype=out_dtype)
    got, got2 = host(dw), host(again)
    assert np.array_equal(got, got2), "split reduction must be deterministic"
    odyt, odyts = oracle.quantize_dim1(dy)
    oxt, oxts = oracle.quantize_dim1(x)
    check_mx_wgrad(oracle, got, odyt, odyts, oxt, oxts, offs, G, f"split wgrad {'bf16' if out_dtype else 'f32'}",
                   out_bf16=out_dtype == mx.MX_OUT_BF16)
