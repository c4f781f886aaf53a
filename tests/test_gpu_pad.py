"""GPU parity of token-group padding, and of the grouped GEMM path through it.

Padding and unpadding are row moves: compared bit-exactly with the oracle, every
row of the padded buffer (zero rows included) and the padded offsets, on buffers
pre-filled with a sentinel so that a row the kernel skips shows. The padded MoE
path (pad X and dY, one-pass casts, forward / dgrad / wgrad on the padded offsets,
unpad Y and dX) is compared with the oracle's composition of the same steps:
codes bit-exact, GEMM outputs within the bars of gemm_check.
"""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import synth

import mfma_model
from gemm_check import check_mx, check_mx_fwd, check_mx_wgrad
from gpu_util import dev_bf16, dev_i32, dev_u8, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def offs_of(sizes):
    return np.cumsum(sizes).astype(np.int32)


def random_sizes(rng, total, G, empty=0):
    cuts = np.sort(rng.integers(0, total + 1, size=G - 1))
    sizes = np.diff(np.concatenate([[0], cuts, [total]]))
    for g in rng.choice(G, size=empty, replace=False):
        sizes[(g + 1) % G] += sizes[g]
        sizes[g] = 0
    return sizes


def _many_groups():
    rng = np.random.default_rng(4)
    return random_sizes(rng, 3000, 1024, empty=300).tolist()


PAD_CASES = [
    # rows, cols, row pitch of x, group sizes (their sum may stay below rows)
    (40, 64, 64, [3, 0, 37]),
    (0, 8, 8, [0, 0]),
    (1, 8, 16, [1]),
    (70, 4104, 4104, [33, 32]),  # 513 chunks per row (partial second pass); 5 rows past the groups
    (65, 72, 80, [0, 31, 1, 33]),
    (96, 256, 256, [32, 32, 32]),  # aligned: identity
    (1000, 256, 264, random_sizes(np.random.default_rng(1), 1000, 8, empty=2).tolist()),
    (3000, 128, 128, _many_groups()),  # the largest group count, many empty groups
]


@pytest.mark.parametrize("rows,cols,ld,sizes", PAD_CASES, ids=[f"r{c[0]}c{c[1]}g{len(c[3])}" for c in PAD_CASES])
def test_pad_matches_oracle(oracle, rows, cols, ld, sizes):
    rng = np.random.default_rng(rows + cols)
    offs = offs_of(sizes)
    G = len(sizes)
    x_full = rng.integers(0, 1 << 16, size=(rows, ld), dtype=np.uint64).astype(np.uint16)
    x = x_full[:, :cols]
    rows_pad = mx.mx_padded_rows(rows, G)
    assert rows_pad == oracle.padded_rows(rows, G)
    say(f"[pad] rows={rows} cols={cols} ld={ld} G={G} rows_pad={rows_pad}")
    dx = dev_bf16(x_full)[:, :cols]
    x_pad = torch.full((rows_pad, cols), -1, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    offs_pad = torch.full((G,), -7, dtype=torch.int32, device="cuda:0")
    mx.mx_pad_token_groups(dx, dev_i32(offs), rows_pad, x_pad=x_pad, offs_pad=offs_pad)
    ref, ref_offs = oracle.pad_token_groups(x, offs.tolist(), rows_pad)
    assert host(offs_pad).tolist() == ref_offs
    got = host(x_pad)
    bad = np.nonzero(np.any(got != ref, axis=1))[0]
    assert bad.size == 0, f"{bad.size} padded rows differ, first {bad[:8].tolist()}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols,sizes", [(40, 64, [3, 0, 37]), (70, 1028, [33, 32]),
                                             (1000, 96, random_sizes(np.random.default_rng(2), 1000, 8, 1).tolist())])
def test_unpad_matches_oracle(oracle, dtype, rows, cols, sizes):
    if dtype == torch.bfloat16 and cols % 8:
        cols += 8 - cols % 8
    rng = np.random.default_rng(rows * 7 + cols)
    offs = offs_of(sizes)
    G = len(sizes)
    rows_pad = mx.mx_padded_rows(rows, G)
    y_pad = torch.from_numpy(rng.standard_normal((rows_pad, cols)).astype(np.float32)).to("cuda:0").to(dtype)
    sentinel = torch.full((rows, cols), 12345.0, dtype=dtype, device="cuda:0")
    say(f"[unpad] rows={rows} cols={cols} G={G} dtype={dtype}")
    y = host(mx.mx_unpad_token_groups(y_pad, dev_i32(offs), rows, y=sentinel.clone())).view(np.uint8)
    src = host(y_pad).view(np.uint8)
    ref = oracle.unpad_token_groups(src, offs.tolist(), rows)
    grouped = int(offs[-1])
    assert np.array_equal(y[:grouped], ref[:grouped])
    assert np.array_equal(y[grouped:], host(sentinel).view(np.uint8)[grouped:])


def test_pad_full_size(oracle):
    """The MoE token tensor (16384 x 4096, 8 experts) with unaligned multinomial group sizes."""
    M, K, G = 16384, 4096, 8
    rng = np.random.default_rng(16384)
    sizes = rng.multinomial(M, np.full(G, 1.0 / G))
    offs = offs_of(sizes)
    x = synth.normal_bf16(rng, (M, K), 1.0)
    rows_pad = mx.mx_padded_rows(M, G)
    say(f"[pad full] sizes={sizes.tolist()} rows_pad={rows_pad}")
    x_pad, offs_pad = mx.mx_pad_token_groups(dev_bf16(x), dev_i32(offs))
    ref, ref_offs = oracle.pad_token_groups(x, offs.tolist(), rows_pad)
    assert host(offs_pad).tolist() == ref_offs
    assert np.array_equal(host(x_pad), ref)
    y = mx.mx_unpad_token_groups(x_pad, dev_i32(offs), M)
    assert np.array_equal(host(y), x)


@pytest.mark.parametrize("M,N,K,sizes", [
    (600, 192, 256, [100, 0, 37, 200, 263]),
    (1000, 128, 576, random_sizes(np.random.default_rng(3), 1000, 6, 1).tolist()),
])
def test_padded_moe_path(oracle, M, N, K, sizes):
    """pad -> one-pass casts -> fwd / dgrad / wgrad on padded offsets -> unpad."""
    rng = np.random.default_rng(M + N + K)
    G = len(sizes)
    offs = offs_of(sizes)
    x = synth.normal_bf16(rng, (M, K), 1.0)
    w = synth.normal_bf16(rng, (G, N, K), 0.02)
    dy = synth.normal_bf16(rng, (M, N), 1e-2)
    rows_pad = mx.mx_padded_rows(M, G)
    say(f"[padded path] M={M} N={N} K={K} sizes={sizes} rows_pad={rows_pad}")
    doffs = dev_i32(offs)
    x_pad, offs_pad = mx.mx_pad_token_groups(dev_bf16(x), doffs)
    dy_pad, _ = mx.mx_pad_token_groups(dev_bf16(dy), doffs)
    xq, xs, xtq, xts = mx.mx_quantize_dim0_dim1(x_pad)
    dyq, dys, dytq, dyts = mx.mx_quantize_dim0_dim1(dy_pad)
    wq, ws = mx.mx_quantize_dim0(dev_bf16(w.reshape(G * N, K)))
    wtq, wts = mx.mx_quantize_dim1(dev_bf16(w))
    y = mx.mx_unpad_token_groups(
        mx.mx_grouped_mm_fwd(xq, xs, wq, ws, offs_pad, rows_pad, N, K, groups=G, out_dtype=mx.MX_OUT_F32), doffs, M)
    dx = mx.mx_unpad_token_groups(
        mx.mx_grouped_mm_dgrad(dyq, dys, wtq, wts, offs_pad, rows_pad, N, K, groups=G, out_dtype=mx.MX_OUT_F32),
        doffs, M)
    dw = mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, offs_pad, rows_pad, N, K, groups=G, out_dtype=mx.MX_OUT_F32)

    ox_pad, ooffs_pad = oracle.pad_token_groups(x, offs.tolist(), rows_pad)
    ody_pad, _ = oracle.pad_token_groups(dy, offs.tolist(), rows_pad)
    assert host(offs_pad).tolist() == ooffs_pad
    oxq, oxs = oracle.quantize_dim0(ox_pad)
    oxt, oxts = oracle.quantize_dim1(ox_pad)
    odyq, odys = oracle.quantize_dim0(ody_pad)
    odyt, odyts = oracle.quantize_dim1(ody_pad)
    assert np.array_equal(host(xq), oxq) and np.array_equal(host(xtq), oxt)
    assert np.array_equal(host(dyq), odyq) and np.array_equal(host(dytq), odyt)
    owq, ows = oracle.quantize_dim0(w.reshape(G * N, K))
    parts = [oracle.quantize_dim1(w[g]) for g in range(G)]
    owt, owts = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])

    def unpadded_check(got, aq, as_, bq, bs, name, k_len):
        # the padded GEMM, then the unpad gather, against the oracle and the MFMA model
        unpad = lambda t: oracle.unpad_token_groups(t, offs.tolist(), M)  # noqa: E731
        ref = unpad(oracle.mx_grouped_mm_fwd(aq, as_, bq, bs, ooffs_pad, G))
        h, ab = mfma_model.grouped_fwd(aq, as_, bq, bs, ooffs_pad, G)
        bound = mfma_model.grouped_fwd(aq, as_, bq, bs, ooffs_pad, G, fn=mfma_model.run_bound_mm)
        check_mx(oracle, got, ref, unpad(ab), k_len, name, h=unpad(h), bound=unpad(bound))

    unpadded_check(host(y), oxq, oxs, owq, ows, "padded fwd", K)
    unpadded_check(host(dx), odyq, odys, owt, owts, "padded dgrad", N)
    check_mx_wgrad(oracle, host(dw), odyt, odyts, oxt, oxts, ooffs_pad, G, "padded wgrad")


def exact_operands(rng, rows, k):
    choices = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], np.uint8)
    return rng.choice(choices, size=(rows, k)), rng.integers(126, 129, size=(rows, k // 32)).astype(np.uint8)


def test_gemm_rows_past_last_group(oracle):
    """offs[G-1] < m: forward leaves the rows past the last group unwritten and
    wgrad does not read the tokens there (they hold non-zero codes here)."""
    rng = np.random.default_rng(9)
    m, n, k, sizes = 320, 96, 256, [64, 0, 96]
    G = len(sizes)
    offs = offs_of(sizes)
    a_q, a_s = exact_operands(rng, m, k)
    b_q, b_s = exact_operands(rng, G * n, k)
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    say("[gemm rows past last group] fwd")
    mx.mx_grouped_mm_fwd(dev_u8(a_q), dev_u8(oracle.scales_to_physical(a_s)), dev_u8(b_q),
                         dev_u8(oracle.scales_to_physical(b_s)), dev_i32(offs), m, n, k, groups=G,
                         out_dtype=mx.MX_OUT_F32, out=out)
    got = host(out)
    ref = oracle.mx_grouped_mm_fwd(a_q, a_s, b_q, b_s, offs, G)
    assert np.array_equal(got[:offs[-1]], ref[:offs[-1]].astype(np.float32))
    assert np.all(np.isnan(got[offs[-1]:]))
    say("[gemm rows past last group] wgrad")
    dy_t, dy_ts = exact_operands(rng, n, m)
    x_t, x_ts = exact_operands(rng, k, m)
    dw = mx.mx_grouped_mm_wgrad(dev_u8(dy_t), dev_u8(oracle.scales_to_physical(dy_ts)), dev_u8(x_t),
                                dev_u8(oracle.scales_to_physical(x_ts)), dev_i32(offs), m, n, k, groups=G,
                                out_dtype=mx.MX_OUT_F32)
    assert np.array_equal(host(dw), oracle.mx_grouped_mm_wgrad(dy_t, dy_ts, x_t, x_ts, offs, G).astype(np.float32))


FUSED_CASES = [
    (600, 256, 256, [100, 0, 37, 200, 263]),
    (70, 288, 320, [33, 32]),  # rows past the last group; pitch wider than the row
    (0, 64, 64, [0, 0]),
    (1000, 96, 96, random_sizes(np.random.default_rng(6), 1000, 6, 1).tolist()),
    (3000, 128, 128, _many_groups()),
    # more tiles than compute units (18 x 17): the four-wave workgroups of the bench's size
    (4400, 4160, 4160, random_sizes(np.random.default_rng(9), 4300, 7, 1).tolist()),
]


@pytest.mark.parametrize("stream_t", [False, True], ids=["cached", "stream_t"])
@pytest.mark.parametrize("rows,cols,ld,sizes", FUSED_CASES, ids=[f"r{c[0]}c{c[1]}g{len(c[3])}" for c in FUSED_CASES])
def test_pad_quantize_matches_oracle(oracle, rows, cols, ld, sizes, stream_t):
    """The padded one-pass cast equals the oracle's padding followed by its casts:
    codes, physical scale bytes (pads included) and padded offsets, bit for bit; with
    MX_FORM_STREAM_T (q_t stored past the caches) the same."""
    rng = np.random.default_rng(rows + cols + 11)
    offs = offs_of(sizes)
    G = len(sizes)
    x_full = synth.normal_bf16(rng, (rows, ld), 1.0) if rows else np.zeros((0, ld), np.uint16)
    x = x_full[:, :cols]
    rows_pad = mx.mx_padded_rows(rows, G)
    say(f"[pad+cast] rows={rows} cols={cols} G={G} rows_pad={rows_pad} stream_t={stream_t}")
    q, s, qt, st, offs_pad = mx.mx_pad_quantize_dim0_dim1(dev_bf16(x_full)[:, :cols], dev_i32(offs), stream_t=stream_t)
    x_pad, ref_offs = oracle.pad_token_groups(x, offs.tolist(), rows_pad)
    assert host(offs_pad).tolist() == ref_offs
    oq, os_ = oracle.quantize_dim0(x_pad)
    oqt, ost = oracle.quantize_dim1(x_pad)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(qt), oqt)
    assert np.array_equal(host(s), oracle.scales_to_physical(os_))
    assert np.array_equal(host(st), oracle.scales_to_physical(ost))


@pytest.mark.parametrize("M,N,K,sizes", [
    (600, 192, 256, [100, 0, 37, 200, 263]),
    (1000, 128, 576, random_sizes(np.random.default_rng(3), 1000, 6, 1).tolist()),
    (700, 96, 128, [64, 0, 600]),  # 36 rows past the last group stay untouched
])
def test_padded_gemm_outputs(oracle, M, N, K, sizes):
    """fwd / dgrad on padded rows writing unpadded outputs equal the unpadded
    oracle results; rows past the last group are not written."""
    rng = np.random.default_rng(M + K + 5)
    G = len(sizes)
    offs = offs_of(sizes)
    x = synth.normal_bf16(rng, (M, K), 1.0)
    w = synth.normal_bf16(rng, (G, N, K), 0.02)
    dy = synth.normal_bf16(rng, (M, N), 1e-2)
    rows_pad = mx.mx_padded_rows(M, G)
    say(f"[padded gemm] M={M} N={N} K={K} sizes={sizes}")
    doffs = dev_i32(offs)
    xq, xs, _, _, offs_pad = mx.mx_pad_quantize_dim0_dim1(dev_bf16(x), doffs)
    dyq, dys, _, _, _ = mx.mx_pad_quantize_dim0_dim1(dev_bf16(dy), doffs)
    wq, ws = mx.mx_quantize_dim0(dev_bf16(w.reshape(G * N, K)))
    wtq, wts = mx.mx_quantize_dim1(dev_bf16(w))
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    dx = torch.full((M, K), float("nan"), dtype=torch.float32, device="cuda:0")
    mx.mx_grouped_mm_fwd_padded(xq, xs, wq, ws, offs_pad, doffs, rows_pad, M, N, K, out_dtype=mx.MX_OUT_F32, out=y)
    mx.mx_grouped_mm_dgrad_padded(dyq, dys, wtq, wts, offs_pad, doffs, rows_pad, M, N, K, out_dtype=mx.MX_OUT_F32,
                                  out=dx)
    grouped = int(offs[-1])
    oxq, oxs = oracle.quantize_dim0(x)
    owq, ows = oracle.quantize_dim0(w.reshape(G * N, K))
    gy, gdx = host(y), host(dx)
    check_mx_fwd(oracle, gy, oxq, oxs, owq, ows, offs, G, "fwd padded->unpadded")
    odyq, odys = oracle.quantize_dim0(dy)
    parts = [oracle.quantize_dim1(w[g]) for g in range(G)]
    owt, owts = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    check_mx_fwd(oracle, gdx, odyq, odys, owt, owts, offs, G, "dgrad padded->unpadded")
    assert np.all(np.isnan(gy[grouped:])) and np.all(np.isnan(gdx[grouped:]))
