"""Pins for the oracle's backward override arms (CPU only).

The arms (ao fork PR 10, "Design notes"): "high_precision" takes both gradients
from the saved bf16 operands through bf16 grouped GEMMs; "dequantized" from the
forward's quantized operands dequantized to bf16. Pinned by an independent integer
construction of every dequantized bf16 value, brute-force loops on tiny grouped
cases, the lossless case where both arms must agree exactly, and the size of the
gap between the arms that the page reports (about 5%, under a 0.15 bound).
"""

import numpy as np
import pytest

from mxfp8_block_scaled_amd import synth


def bf16_by_fields(code, byte):
    """Dequantized bf16 bits of one E4M3 code at scale byte `byte`, built from the
    fields: value = (1 + m/8) 2^(e-7) (e > 0) or m 2^-9 (e = 0), times 2^(byte-127),
    then placed in bf16's fields, rounding to nearest even below 2^-126."""
    sign = (code >> 7) & 1
    e, m = (code >> 3) & 15, code & 7
    if e == 0 and m == 0:
        return sign << 15
    # as an integer significand f times 2^x: f in [8, 16)
    if e == 0:
        f, x = m, -9
        while f < 8:
            f, x = f * 2, x - 1
        x += 3  # f = m * 2^k scaled so value = f * 2^(x - 3)
    else:
        f, x = 8 + m, e - 7
    x += byte - 127  # value = f * 2^(x - 3), f in [8, 16)
    biased = x + 127
    if biased >= 255:
        return (sign << 15) | 0x7F80
    if biased >= 1:
        return (sign << 15) | (biased << 7) | ((f - 8) << 4)
    # subnormal: value / 2^-133 = f * 2^(x - 3 + 133), rounded to an integer
    shift = x + 130
    if shift >= 0:
        q = f << shift
    else:
        k = -shift
        q, r = f >> k, f & ((1 << k) - 1)
        half = 1 << (k - 1)
        if r > half or (r == half and q & 1):
            q += 1
    return (sign << 15) | q


def test_dequantize_to_bf16_every_code_and_scale(oracle):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    for byte in range(0, 255):
        q = np.zeros((1, 256), np.uint8)
        q[0, :codes.size] = codes
        got = oracle.dequantize_to_bf16_bits(q, np.full((1, 8), byte, np.uint8))[0, :codes.size]
        want = np.array([bf16_by_fields(int(c), byte) for c in codes], np.uint16)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"byte {byte}: code {codes[bad[0]]:#04x} -> {got[bad[0]]:#06x}, want {want[bad[0]]:#06x}"


def test_field_construction_spot_values():
    """Hand-checked values of the independent construction itself."""
    assert bf16_by_fields(0x38, 127) == 0x3F80  # 1.0
    assert bf16_by_fields(0x7E, 127) == 0x43E0  # 448
    assert bf16_by_fields(0xB8, 128) == 0xC000  # -1 * 2 = -2
    assert bf16_by_fields(0x01, 127) == 0x3B00  # 2^-9
    assert bf16_by_fields(0x08, 0) == 0x0001  # 2^-6 * 2^-127 = 2^-133, the smallest bf16
    assert bf16_by_fields(0x04, 0) == 0x0000  # 2^-7 * 2^-127 = 2^-134: a tie, to even (0)
    assert bf16_by_fields(0x0C, 0) == 0x0002  # 1.5 * 2^-133: a tie between 1 and 2 -> 2
    assert bf16_by_fields(0x7E, 247) == 0x7F80  # 1.75 * 2^128: above the largest bf16


def brute_backward(x, w, dy, offs, G):
    M, K = x.shape
    N = w.shape[0] // G
    dx = np.zeros((M, K))
    dw = np.zeros((G, N, K))
    starts = [0] + list(offs[:-1])
    for g in range(G):
        for r in range(starts[g], offs[g]):
            for kk in range(K):
                dx[r, kk] = sum(dy[r, n] * w[g * N + n, kk] for n in range(N))
        for n in range(N):
            for kk in range(K):
                dw[g, n, kk] = sum(dy[r, n] * x[r, kk] for r in range(starts[g], offs[g]))
    return dx, dw


def test_backward_matches_loops(oracle):
    rng = np.random.default_rng(0)
    M, N, K, G = 11, 3, 4, 3
    offs = [4, 4, 11]  # unaligned, one empty group
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((G * N, K))
    dy = rng.standard_normal((M, N))
    dx, dw = oracle.backward_bf16(x, w, dy, offs, G)
    bdx, bdw = brute_backward(x, w, dy, offs, G)
    np.testing.assert_allclose(dx, bdx, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, bdw, rtol=1e-12, atol=1e-12)
    assert not dw[1].any()


def representable(rng, rows, cols):
    """bf16 blocks that quantize losslessly: E4M3 code values (|v| in (224, 448] at
    the block maximum) times 2^s, so dequantize(quantize(x)) == x."""
    codes = rng.integers(0, 0x7F, size=(rows, cols)).astype(np.uint8) | (rng.integers(0, 2, (rows, cols)) << 7).astype(np.uint8)
    codes[:, ::32] = 0x7A  # 320: puts every block maximum in (224, 448]
    s = rng.integers(110, 135, size=(rows, cols // 32))
    from oracle import mx
    vals = mx.e4m3_decode(codes) * np.repeat(np.ldexp(1.0, s - 127), 32, axis=1)
    return mx.round_to_bf16_bits(vals)


def test_arms_agree_on_lossless_operands(oracle):
    """When X and W are exactly representable per block, quantize-then-dequantize
    returns them unchanged, so the dequantized arm equals the high-precision arm."""
    rng = np.random.default_rng(1)
    M, N, K, G = 96, 64, 128, 3
    offs = [32, 32, 96]
    x = representable(rng, M, K)
    w = representable(rng, G * N, K)
    dy = synth.normal_bf16(rng, (M, N), 1e-2)
    xq, xs = oracle.quantize_dim0(x)
    wq, ws = oracle.quantize_dim0(w)
    assert np.array_equal(oracle.dequantize_to_bf16_bits(xq, xs), x)
    hp = oracle.backward_high_precision(x, w, dy, offs, G)
    dq = oracle.backward_dequantized(xq, xs, wq, ws, dy, offs, G)
    assert np.array_equal(hp[0], dq[0]) and np.array_equal(hp[1], dq[1])


def test_arms_gap_matches_the_pages_evidence(oracle):
    """On N(0,1) tokens and N(0,0.02) weights the two arms' gradients differ by a
    few percent (the page observes about 5% and tests against 0.15)."""
    rng = np.random.default_rng(2)
    M, N, K, G = 512, 128, 256, 4
    offs = [100, 200, 380, 512]
    x = synth.normal_bf16(rng, (M, K), 1.0)
    w = synth.normal_bf16(rng, (G * N, K), 0.02)
    dy = synth.normal_bf16(rng, (M, N), 1e-2)
    xq, xs = oracle.quantize_dim0(x)
    wq, ws = oracle.quantize_dim0(w)
    hp = oracle.backward_high_precision(x, w, dy, offs, G)
    dq = oracle.backward_dequantized(xq, xs, wq, ws, dy, offs, G)
    for name, a, b in (("dX", dq[0], hp[0]), ("dW", dq[1], hp[1])):
        rel = oracle.rel_frobenius(a, b)
        assert 0.005 < rel < 0.15, (name, rel)


@pytest.mark.parametrize("G", [1, 4])
def test_dgrad_uses_each_groups_weight(oracle, G):
    """Permuting the groups (rows and weights together) permutes dX rows and dW."""
    rng = np.random.default_rng(3)
    N, K = 8, 16
    sizes = rng.integers(1, 9, size=G)
    offs = list(np.cumsum(sizes))
    M = offs[-1]
    x, dy = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    w = rng.standard_normal((G * N, K))
    dx, dw = oracle.backward_bf16(x, w, dy, offs, G)
    perm = rng.permutation(G)
    starts = [0] + offs[:-1]
    rows = np.concatenate([np.arange(starts[g], offs[g]) for g in perm])
    w_p = np.concatenate([w[g * N:(g + 1) * N] for g in perm])
    offs_p = list(np.cumsum(sizes[perm]))
    dx_p, dw_p = oracle.backward_bf16(x[rows], w_p, dy[rows], offs_p, G)
    np.testing.assert_allclose(dx_p, dx[rows], rtol=1e-12)
    np.testing.assert_allclose(dw_p, dw[perm], rtol=1e-12)
