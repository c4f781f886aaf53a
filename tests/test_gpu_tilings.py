"""GPU parity of every GEMM tile configuration, full outputs against the oracle.

The library picks a tiling from the problem's shape; each case here is shaped to
select one of them, with groups that end inside tiles (MXFP8 groups on 32-row
boundaries, as the calls require; bf16 groups anywhere), one group empty, and
partial tiles on both output edges:
  * 256x256 with eight waves (two per SIMD): 256..511 tiles of 256x256 (M-grouped
    over a contraction above 1024), K-grouped wgrads of 256 or more such tiles, and
    M-grouped fp32 outputs with more tiles;
  * 128x256 over a three-deep ring, two blocks per compute unit: M-grouped with a
    contraction of at most 1024 and >= 128 tiles, and either mode with 128..255
    tiles of 256x256 (half a round to a round);
  * 192x256: K-grouped outputs whose rows 192-row tiles cover with at least 1/8
    less padding than 256-row ones, without and with split contractions;
  * 256x192: M-grouped outputs whose columns 192-column tiles cover with at least
    1/8 less padding (96-column waves: the epilogue's padded-pitch staging).
The bit-exact sweep below also reaches 128x128 and the four-wave 256x256 (M-grouped
bf16 output, 512 or more tiles), which the small-shape and full-size tests cover too, and
the split of a short last round of 256x256 tiles into 128x128 quarters.
"""

import numpy as np
import pytest

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import synth

from gemm_check import check_bf16, check_f32, check_mx_fwd, check_mx_wgrad
from gpu_util import dev_bf16, dev_i32, dev_u8, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def fwd_case(oracle, m, n, k, sizes, seed, name):
    """M-grouped forward, fp32 and bf16 outputs, against the oracle's product of the
    oracle's own casts (the casts are bit-exact, tested elsewhere)."""
    rng = np.random.default_rng(seed)
    G = len(sizes)
    offs = synth.offs_from_sizes(np.array(sizes))
    x = synth.normal_bf16(rng, (m, k), 1.0)
    w = synth.normal_bf16(rng, (G * n, k), 0.02)
    say(f"[tiling {name}] fwd m={m} n={n} k={k} offs={offs.tolist()}")
    xq, xs = mx.mx_quantize_dim0(dev_bf16(x))
    wq, ws = mx.mx_quantize_dim0(dev_bf16(w))
    doffs = dev_i32(offs)
    got = host(mx.mx_grouped_mm_fwd(xq, xs, wq, ws, doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
    got16 = host(mx.mx_grouped_mm_fwd(xq, xs, wq, ws, doffs, m, n, k, out_dtype=mx.MX_OUT_BF16))
    oxq, oxs = oracle.quantize_dim0(x)
    owq, ows = oracle.quantize_dim0(w)
    # the model on the rows at every group edge and a random sample
    edges = np.concatenate([[0], offs[:-1], np.maximum(offs - 1, 0)])
    mrows = np.unique(np.concatenate([edges, rng.integers(0, m, 40)]))
    check_mx_fwd(oracle, got, oxq, oxs, owq, ows, offs, G, f"{name} fwd f32", model_rows=mrows)
    check_mx_fwd(oracle, got16, oxq, oxs, owq, ows, offs, G, f"{name} fwd bf16", out_bf16=True, model_rows=mrows)
    return offs, rng


def wgrad_case(oracle, n, k, m, sizes, seed, name):
    """K-grouped wgrad (dw[g] = dy_t[:, rows_g] . x_t[:, rows_g]^T), fp32 and bf16."""
    rng = np.random.default_rng(seed)
    G = len(sizes)
    offs = synth.offs_from_sizes(np.array(sizes))
    dy = synth.normal_bf16(rng, (m, n), 1e-2)
    x = synth.normal_bf16(rng, (m, k), 1.0)
    say(f"[tiling {name}] wgrad n={n} k={k} m={m} offs={offs.tolist()}")
    dytq, dyts = mx.mx_quantize_dim1(dev_bf16(dy))
    xtq, xts = mx.mx_quantize_dim1(dev_bf16(x))
    doffs = dev_i32(offs)
    got = host(mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
    got16 = host(mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, doffs, m, n, k, out_dtype=mx.MX_OUT_BF16))
    odyt, odyts = oracle.quantize_dim1(dy)
    oxt, oxts = oracle.quantize_dim1(x)
    mrows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 14)]))
    check_mx_wgrad(oracle, got, odyt, odyts, oxt, oxts, offs, G, f"{name} wgrad f32", model_rows=mrows)
    check_mx_wgrad(oracle, got16, odyt, odyts, oxt, oxts, offs, G, f"{name} wgrad bf16", out_bf16=True,
                   model_rows=mrows)


def test_mgroup_eight_waves(oracle):
    """16 x 16 = 256 tiles of 256x256 over K = 1280: the eight-wave tiling."""
    fwd_case(oracle, 4000, 4064, 1280, [992, 0, 1504, 1504], 61, "8-wave")


def test_mgroup_half_round(oracle):
    """16 x 9 = 144 tiles of 256x256 over K = 1280 (less than a round): 128x256 tiles."""
    fwd_case(oracle, 4000, 2080, 1280, [992, 0, 1504, 1504], 60, "128x256 half round")


def test_mgroup_short_contraction(oracle):
    """K = 576 with 128 tiles: 128x256 tiles, two blocks per compute unit; grouped and
    dense, and the dgrad form (contraction over the 576 output columns of the forward)."""
    fwd_case(oracle, 4000, 2016, 576, [992, 0, 1504, 1504], 62, "128x256 grouped")
    fwd_case(oracle, 4000, 2016, 576, [4000], 63, "128x256 dense")
    rng = np.random.default_rng(64)
    m, n, k, sizes = 4000, 576, 2016, [1504, 992, 0, 1504]
    G = len(sizes)
    offs = synth.offs_from_sizes(np.array(sizes))
    dy = synth.normal_bf16(rng, (m, n), 1e-2)
    w_t = synth.normal_bf16(rng, (G * k, n), 0.02)
    say(f"[tiling 128x256] dgrad m={m} n={n} k={k} offs={offs.tolist()}")
    dyq, dys = mx.mx_quantize_dim0(dev_bf16(dy))
    wtq, wts = mx.mx_quantize_dim0(dev_bf16(w_t))
    got = host(mx.mx_grouped_mm_dgrad(dyq, dys, wtq, wts, dev_i32(offs), m, n, k, out_dtype=mx.MX_OUT_F32))
    odyq, odys = oracle.quantize_dim0(dy)
    owtq, owts = oracle.quantize_dim0(w_t)
    edges = np.concatenate([[0], offs[:-1], np.maximum(offs - 1, 0)])
    mrows = np.unique(np.concatenate([edges, rng.integers(0, m, 40)]))
    check_mx_fwd(oracle, got, odyq, odys, owtq, owts, offs, G, "128x256 dgrad f32", model_rows=mrows)


def test_kgroup_eight_waves(oracle):
    """992 x 2080 outputs per group, 8 groups (one empty): 4 x 9 x 8 = 288 tiles."""
    wgrad_case(oracle, 992, 2080, 4096, [640, 512, 0, 736, 480, 576, 608, 544], 65, "8-wave")


def test_kgroup_half_round(oracle):
    """992 x 1056 outputs per group, 8 groups (one empty): 4 x 5 x 8 = 160 tiles of
    256x256, less than a round: 128x256 tiles, the contraction not split."""
    wgrad_case(oracle, 992, 1056, 4096, [640, 512, 0, 736, 480, 576, 608, 544], 64, "128x256 half round")


def test_kgroup_192_row_tiles(oracle):
    """352-row outputs (two 192-row tiles, the second partial) x 2016 columns, 8 groups."""
    wgrad_case(oracle, 352, 2016, 4096, [480, 0, 640, 512, 736, 544, 608, 576], 66, "192x256")


def test_kgroup_192_row_tiles_split(oracle):
    """576 x 1024 outputs over 16384 tokens in one group: 12 output tiles, so the
    contraction is split 16 ways (192x256 tiles, fp32 partials summed in order)."""
    wgrad_case(oracle, 576, 1024, 16384, [16384], 67, "192x256 split")


@pytest.mark.parametrize("sizes", [[1001, 0, 1999, 1096], [4095, 0, 0, 1]])
def test_bf16_tilings(oracle, sizes):
    """bf16 operands through the eight-wave (forward K=1280; wgrad, 128 tiles so its
    contraction splits two ways) and 128x256 (forward K=576) tilings; token groups end
    off 8-element boundaries, so the wgrad masks group edges inside 16-byte chunks."""
    rng = np.random.default_rng(sum(sizes))
    G = len(sizes)
    m = int(sum(sizes))
    offs = synth.offs_from_sizes(np.array(sizes))
    doffs = dev_i32(offs)
    for n, k, name in ((4064, 1280, "8-wave"), (2016, 576, "128x256")):
        a = synth.normal_bf16(rng, (m, k), 1.0)
        b = synth.normal_bf16(rng, (G * n, k), 0.02)
        say(f"[tiling bf16 {name}] fwd m={m} n={n} k={k} offs={offs.tolist()}")
        got = host(mx.mx_grouped_mm_bf16_fwd(dev_bf16(a), dev_bf16(b), doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
        fa, fb = oracle.bf16_to_f64(a), oracle.bf16_to_f64(b)
        check_f32(oracle, got, oracle.grouped_mm(fa, fb, offs, G), f"bf16 {name} fwd f32",
                  oracle.grouped_mm(np.abs(fa), np.abs(fb), offs, G), k)
    n, k = 1000, 2000
    dy = synth.normal_bf16(rng, (m, n), 1e-2)
    x = synth.normal_bf16(rng, (m, k), 1.0)
    say(f"[tiling bf16 8-wave] wgrad n={n} k={k} m={m}")
    dw = host(mx.mx_grouped_mm_bf16_wgrad(dev_bf16(np.ascontiguousarray(dy.T)), dev_bf16(np.ascontiguousarray(x.T)),
                                          doffs, m, n, k, out_dtype=mx.MX_OUT_F32))
    fdy, fx = oracle.bf16_to_f64(dy), oracle.bf16_to_f64(x)
    check_f32(oracle, dw, oracle.grouped_mm_wgrad(fdy.T, fx.T, offs, G), "bf16 8-wave wgrad f32",
              oracle.grouped_mm_wgrad(np.abs(fdy).T, np.abs(fx).T, offs, G), int(max(sizes)))
    for g in np.flatnonzero(np.array(sizes) == 0):
        assert not dw[g].any()


# ---- bit-exact sweep -------------------------------------------------------------------
# Codes in {0, +-0.5, +-1, +-2} with scales 2^-1..2^1: every product is a power of two in
# [2^-4, 2^4] and every partial sum is exact in fp32, so each tiling must reproduce the
# oracle bit for bit: fp32 outputs equal the exact sums, bf16 outputs their correctly
# rounded value. Large cases compare a seeded sample of output rows.

def exact_codes(rng, rows, k):
    choices = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], np.uint8)
    return rng.choice(choices, size=(rows, k)), rng.integers(126, 129, size=(rows, k // 32)).astype(np.uint8)


def phys(oracle, logical):
    return dev_u8(oracle.scales_to_physical(logical))


def random_sizes(rng, total, groups):
    """Group sizes in 32-row units summing to `total`, one group forced empty."""
    units = rng.multinomial(total // 32, np.full(groups, 1.0 / groups))
    units[rng.integers(groups)] = 0
    units[rng.integers(groups)] += total // 32 - units.sum()
    return units * 32


def sample_rows(rng, upto, count):
    return np.sort(rng.choice(upto, size=min(count, upto), replace=False))


@pytest.mark.parametrize("m,n,k,G,name", [
    (4128, 4640, 1280, 3, "8-wave"),        # 17 x 19 = 323 tiles, K > 1024
    (4096, 2080, 1280, 3, "128x256 half"),  # 16 x 9 = 144 tiles: less than a round
    (3104, 2336, 576, 3, "128x256"),        # K <= 1024
    (8192, 4128, 1088, 4, "256x256"),       # 32 x 17 = 544 tiles (bf16 out; fp32: 8-wave)
    (1000, 800, 320, 3, "128x128"),         # 4 x 4 tiles
    (16384, 576, 1280, 2, "256x192"),       # 64 x 3 tiles of 256 x 192: 96-column waves
    (16384, 352, 1088, 2, "256x192 ragged"),  # 64 x 2, the second column tile partial
])
def test_exact_fwd_tilings(oracle, m, n, k, G, name):
    rng = np.random.default_rng(m + n + k)
    used = m - 96  # rows past the last group are not written
    sizes = random_sizes(rng, used // 32 * 32, G)
    offs = np.cumsum(sizes).astype(np.int32)
    a, a_s = exact_codes(rng, m, k)
    b, b_s = exact_codes(rng, G * n, k)
    say(f"[exact {name}] fwd m={m} n={n} k={k} offs={offs.tolist()}")
    args = (dev_u8(a), phys(oracle, a_s), dev_u8(b), phys(oracle, b_s), dev_i32(offs), m, n, k)
    got = host(mx.mx_grouped_mm_fwd(*args, out_dtype=mx.MX_OUT_F32))
    got16 = host(mx.mx_grouped_mm_fwd(*args, out_dtype=mx.MX_OUT_BF16))
    rows = sample_rows(rng, int(offs[-1]), 384)
    sub_offs = np.searchsorted(rows, offs, side="left").astype(np.int32)  # group ends within the sample
    ref = oracle.grouped_mm(oracle.dequantize(a[rows], a_s[rows]), oracle.dequantize(b, b_s), sub_offs, G)
    assert np.array_equal(got[rows], ref.astype(np.float32)), f"{name}: fwd differs from the exact result"
    assert np.array_equal(got16[rows], oracle.round_to_bf16_bits(ref)), f"{name}: bf16 fwd is not the rounded exact result"


@pytest.mark.parametrize("n,k,m,G,name", [
    (352, 2080, 4096, 8, "192x256"),        # 8 x 2 x 9 = 144 tiles, 352 rows in 192-row tiles
    (1056, 2080, 4096, 8, "8-wave"),        # 8 x 5 x 9 = 360 tiles (1152 rows as 192s: too little saved)
    (1056, 1056, 4096, 8, "128x256 half"),  # 8 x 5 x 5 = 200 tiles: less than a round, no split
    (4128, 2080, 2048, 8, "256x256"),       # 8 x 17 x 9 = 1224 tiles, eight waves
    (576, 1056, 8192, 2, "192x256 split"),  # 2 x 3 x 5 = 30 tiles: contraction split 8 ways
])
def test_exact_wgrad_tilings(oracle, n, k, m, G, name):
    rng = np.random.default_rng(n + k + m + G)
    sizes = random_sizes(rng, m, G)
    offs = np.cumsum(sizes).astype(np.int32)
    a, a_s = exact_codes(rng, n, m)
    b, b_s = exact_codes(rng, k, m)
    say(f"[exact {name}] wgrad n={n} k={k} m={m} offs={offs.tolist()}")
    args = (dev_u8(a), phys(oracle, a_s), dev_u8(b), phys(oracle, b_s), dev_i32(offs), m, n, k)
    got = host(mx.mx_grouped_mm_wgrad(*args, out_dtype=mx.MX_OUT_F32))
    got16 = host(mx.mx_grouped_mm_wgrad(*args, out_dtype=mx.MX_OUT_BF16))
    rows = sample_rows(rng, n, 160)
    ref = oracle.grouped_mm_wgrad(oracle.dequantize(a[rows], a_s[rows]), oracle.dequantize(b, b_s), offs, G)
    assert np.array_equal(got[:, rows], ref.astype(np.float32)), f"{name}: wgrad differs from the exact result"
    assert np.array_equal(got16[:, rows], oracle.round_to_bf16_bits(ref)), f"{name}: bf16 wgrad is not the rounded exact result"
    for g in np.flatnonzero(sizes == 0):
        assert not got[g].any() and not got16[g].any()


@pytest.mark.parametrize("sizes,n,rest", [
    ([3008, 2912, 2720], 4096, 6),       # 35 x 16 = 560 tiles, 70 per XCD: 64 + 6 left, one quarter per unit
    ([3008, 0, 2912, 2720], 4128, 11),   # 35 x 17 = 595, 75 per XCD (70 on the last): 64 + 11, two quarters
                                         # on some units; ragged last column, an empty group
    ([2560, 2560, 2560, 2560], 4096, 16),  # 40 x 16 = 640, 80 per XCD: 64 + 16, the largest rest split
    ([2048, 2048, 2048, 2048], 4096, 0),   # 32 x 16 = 512: whole rounds, the quarter launch does nothing
    ([2592, 2592, 2592, 2304], 4096, 20),  # 42 x 16 = 672, 84 per XCD: 20 left, more than half a round: no split
])
def test_exact_fwd_last_round_quarters(oracle, sizes, n, rest):
    """M-grouped forward with bf16 output over 256x256 tiles: each XCD's whole rounds
    (32 compute units) run as 256x256 tiles, a short rest as 128x128 quarters in a
    second launch. Every output row is compared with the exact sum, fp32 and bf16."""
    rng = np.random.default_rng(len(sizes) * 1000 + n + rest)
    sizes = np.array(sizes)
    G, m, k = len(sizes), int(sizes.sum()), 1088
    per = (int(np.sum((sizes + 255) // 256)) * ((n + 255) // 256) + 7) // 8
    assert per % 32 == rest
    offs = np.cumsum(sizes).astype(np.int32)
    a, a_s = exact_codes(rng, m, k)
    b, b_s = exact_codes(rng, G * n, k)
    say(f"[exact quarters] fwd m={m} n={n} k={k} offs={offs.tolist()} rest per XCD={rest}")
    args = (dev_u8(a), phys(oracle, a_s), dev_u8(b), phys(oracle, b_s), dev_i32(offs), m, n, k)
    got16 = host(mx.mx_grouped_mm_fwd(*args, out_dtype=mx.MX_OUT_BF16))
    got = host(mx.mx_grouped_mm_fwd(*args, out_dtype=mx.MX_OUT_F32))
    ref = oracle.grouped_mm(oracle.dequantize(a, a_s), oracle.dequantize(b, b_s), offs, G)
    assert np.array_equal(got16, oracle.round_to_bf16_bits(ref)), "bf16 fwd is not the rounded exact result"
    assert np.array_equal(got, ref.astype(np.float32)), "fp32 fwd differs from the exact result"


def test_exact_bf16_fwd_last_round_quarters(oracle):
    """bf16 operands, bf16 output over 256x256 tiles with a short last round (70 tiles per
    XCD: 64 + 6, run as 128x128 quarters): values in {0, +-0.5, +-1, +-2}, so every sum is
    exact in fp32 and the output must be the correctly rounded exact sum, every row."""
    rng = np.random.default_rng(77)
    sizes = np.array([3008, 2912, 2720])
    G, m, n, k = len(sizes), int(sizes.sum()), 4096, 1088
    offs = np.cumsum(sizes).astype(np.int32)
    pats = np.array([0x0000, 0x3F00, 0xBF00, 0x3F80, 0xBF80, 0x4000, 0xC000], np.uint16)
    a, b = rng.choice(pats, size=(m, k)), rng.choice(pats, size=(G * n, k))
    say(f"[exact quarters bf16] fwd m={m} n={n} k={k} offs={offs.tolist()}")
    got = host(mx.mx_grouped_mm_bf16_fwd(dev_bf16(a), dev_bf16(b), dev_i32(offs), m, n, k, out_dtype=mx.MX_OUT_BF16))
    ref = oracle.grouped_mm(oracle.bf16_to_f64(a), oracle.bf16_to_f64(b), offs, G)
    assert np.array_equal(got, oracle.round_to_bf16_bits(ref)), "bf16 fwd is not the rounded exact result"


def test_exact_dgrad_short_contraction(oracle):
    """dgrad over a 576-wide contraction, 13 x 10 tiles: 128x256 tiles, two blocks per CU."""
    rng = np.random.default_rng(81)
    m, n, k, G = 3104, 576, 2336, 3
    offs = np.cumsum(random_sizes(rng, m, G)).astype(np.int32)
    dy, dy_s = exact_codes(rng, m, n)
    w_t, w_t_s = exact_codes(rng, G * k, n)
    say(f"[exact 128x256] dgrad m={m} n={n} k={k} offs={offs.tolist()}")
    got = host(mx.mx_grouped_mm_dgrad(dev_u8(dy), phys(oracle, dy_s), dev_u8(w_t), phys(oracle, w_t_s),
                                      dev_i32(offs), m, n, k, out_dtype=mx.MX_OUT_F32))
    ref = oracle.mx_grouped_mm_fwd(dy, dy_s, w_t, w_t_s, offs, G)
    assert np.array_equal(got, ref.astype(np.float32))
