"""Pins for the oracle's token-group padding (CPU only).

Padding moves each group's token rows to a run starting at a multiple of 32 and
zero-fills the rest (pytorch/ao PR 4705, ghstack list: pad/unpad kernels; ao fork
PR 10, "Known follow-ups": padded offsets feed the grouped GEMM). Pinned by
hand-derived cases, an exhaustive check of the static size bound, the inverse
property, and the padded GEMM path against per-group brute force.
"""

import itertools
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "token_group_padding.txt")


def golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        rows, offs, rows_pad, offs_pad, runs = [f.strip() for f in line.split("|")]
        parsed_runs = [tuple(int(v) for v in r.split(":")) for r in runs.split()] if runs else []
        cases.append((int(rows), [int(v) for v in offs.split(",")], int(rows_pad),
                      [int(v) for v in offs_pad.split(",")], parsed_runs))
    return cases


def test_golden_cases(oracle):
    mx = oracle
    for rows, offs, rows_pad, offs_pad, runs in golden_cases():
        case = (rows, offs)
        assert mx.padded_rows(rows, len(offs)) == rows_pad, case
        assert mx.padded_offsets(offs) == offs_pad, case
        x = np.arange(rows * 3, dtype=np.int64).reshape(rows, 3) + 1  # every source row non-zero
        x_pad, got_offs_pad = mx.pad_token_groups(x, offs, rows_pad)
        assert got_offs_pad == offs_pad, case
        expect = np.zeros((rows_pad, 3), dtype=np.int64)
        for dst, src, n in runs:
            expect[dst:dst + n] = x[src:src + n]
        assert np.array_equal(x_pad, expect), case
        # unpad brings the grouped rows back; rows past offs[-1] stay zero
        back = mx.unpad_token_groups(x_pad, offs, rows)
        grouped = offs[-1]
        assert np.array_equal(back[:grouped], x[:grouped]), case
        assert not back[grouped:].any(), case


def test_size_bound_exhaustive(oracle):
    """padded_rows(rows, G) covers every way to split at most `rows` rows into G
    groups; the worst split, for rows >= G, is sizes 1, ..., 1, rows - G + 1 (each
    small group growing by 31), and the bound is rows + 31 G rounded up to 256."""
    mx = oracle
    for G, max_rows in ((1, 100), (2, 100), (3, 70), (4, 40)):
        for rows in range(0, max_rows):
            worst = 0
            for cuts in itertools.combinations_with_replacement(range(rows + 1), G):
                worst = max(worst, mx.padded_offsets(list(cuts))[-1])
            bound = mx.padded_rows(rows, G)
            assert worst <= bound, (rows, G)
            assert bound % 256 == 0 and rows + 31 * G <= bound < rows + 31 * G + 256
            if rows >= G:
                # the closed form of the worst case
                sizes = [1] * (G - 1) + [rows - G + 1]
                worst_closed = 32 * (G - 1) + 32 * ((rows - G + 1 + 31) // 32)
                assert mx.padded_offsets(list(np.cumsum(sizes)))[-1] == worst_closed
                assert worst == worst_closed


def random_offs(rng, rows, G, empty=0):
    cuts = np.sort(rng.integers(0, rows + 1, size=G - 1))
    offs = list(cuts) + [rows]
    for g in rng.choice(G, size=empty, replace=False):
        if g > 0:
            offs[g] = offs[g - 1]
    return [int(v) for v in np.maximum.accumulate(offs)]


@pytest.mark.parametrize("seed", range(5))
def test_pad_properties(oracle, seed):
    mx = oracle
    rng = np.random.default_rng(seed)
    rows, G = int(rng.integers(1, 300)), int(rng.integers(1, 9))
    offs = random_offs(rng, rows, G, empty=int(rng.integers(0, G)))
    rows_pad = mx.padded_rows(rows, G)
    x = rng.integers(1, 1 << 15, size=(rows, 5)).astype(np.uint16)
    x_pad, offs_pad = mx.pad_token_groups(x, offs, rows_pad)
    prev, prev_pad = 0, 0
    for e, pe in zip(offs, offs_pad):
        size, padded = e - prev, pe - prev_pad
        assert pe % 32 == 0 and 0 <= padded - size < 32 and (padded == 0) == (size == 0)
        np.testing.assert_array_equal(x_pad[prev_pad:prev_pad + size], x[prev:e])
        assert not x_pad[prev_pad + size:pe].any()
        prev, prev_pad = e, pe
    assert offs_pad[-1] <= rows_pad and not x_pad[offs_pad[-1]:].any()
    np.testing.assert_array_equal(mx.unpad_token_groups(x_pad, offs, rows), x)


def test_aligned_offsets_are_identity(oracle):
    mx = oracle
    offs = [64, 64, 160, 192]
    x = np.arange(192 * 2).reshape(192, 2) + 1
    x_pad, offs_pad = mx.pad_token_groups(x, offs, mx.padded_rows(192, 4))
    assert offs_pad == offs
    np.testing.assert_array_equal(x_pad[:192], x)
    assert not x_pad[192:].any()


def bf16_normal(rng, shape, sigma):
    f = (rng.standard_normal(shape) * sigma).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_padded_forward_equals_unpadded_rows(oracle):
    """Forward through padding: dim0 blocks are row-local, so unpad(fwd(pad(X)))
    equals the grouped forward on the unaligned offsets directly."""
    mx = oracle
    rng = np.random.default_rng(7)
    M, K, N, G = 150, 64, 32, 4
    offs = [37, 37, 101, 150]
    x = bf16_normal(rng, (M, K), 1.0)
    w = bf16_normal(rng, (G * N, K), 0.02)
    wq, ws = mx.quantize_dim0(w)
    xq, xs = mx.quantize_dim0(x)
    direct = mx.mx_grouped_mm_fwd(xq, xs, wq, ws, offs, G)
    x_pad, offs_pad = mx.pad_token_groups(x, offs, mx.padded_rows(M, G))
    pq, ps = mx.quantize_dim0(x_pad)
    y_pad = mx.mx_grouped_mm_fwd(pq, ps, wq, ws, offs_pad, G)
    np.testing.assert_allclose(mx.unpad_token_groups(y_pad, offs, M), direct, rtol=1e-12, atol=1e-300)


def test_padded_wgrad_equals_per_group_brute_force(oracle):
    """wgrad through padding: the dim1 (token-axis) blocks of the padded operands
    start at each group's first token and the last block of a group is zero-filled;
    computed here group by group from sliced, zero-extended tensors."""
    mx = oracle
    rng = np.random.default_rng(11)
    M, K, N, G = 150, 64, 96, 4
    offs = [37, 37, 101, 150]
    x = bf16_normal(rng, (M, K), 1.0)
    dy = bf16_normal(rng, (M, N), 1.0)
    rows_pad = mx.padded_rows(M, G)
    x_pad, offs_pad = mx.pad_token_groups(x, offs, rows_pad)
    dy_pad, _ = mx.pad_token_groups(dy, offs, rows_pad)
    xtq, xts = mx.quantize_dim1(x_pad)
    dytq, dyts = mx.quantize_dim1(dy_pad)
    got = mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, offs_pad, G)
    start = 0
    for g, end in enumerate(offs):
        size = end - start
        if size == 0:
            assert not got[g].any()
            continue
        n_blk = (size + 31) // 32
        xg = np.zeros((32 * n_blk, K), dtype=np.uint16)
        dyg = np.zeros((32 * n_blk, N), dtype=np.uint16)
        xg[:size], dyg[:size] = x[start:end], dy[start:end]
        a = mx.dequantize(*mx.quantize_dim0(np.ascontiguousarray(dyg.T)))
        b = mx.dequantize(*mx.quantize_dim0(np.ascontiguousarray(xg.T)))
        np.testing.assert_allclose(got[g], a @ b.T, rtol=1e-12, atol=1e-300)
        start = end
