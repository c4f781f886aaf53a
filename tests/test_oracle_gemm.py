"""Pins for the oracle's grouped GEMM, output rounding and metrics.

Checks against brute force (explicit loops, exact rational arithmetic), structural
identities of the grouped GEMM, and hand-computed values.
"""

import fractions
import math

import numpy as np
import pytest

from mxfp8_block_scaled_amd import synth


def naive_grouped(a, b, offs, G):
    M, K = a.shape
    N = b.shape[0] // G
    out = np.zeros((M, N))
    starts = [0] + list(offs[:-1]) if offs is not None else [0]
    ends = list(offs) if offs is not None else [M]
    for g in range(len(ends)):
        for r in range(starts[g], ends[g]):
            for n in range(N):
                s = 0.0
                for k in range(K):
                    s += a[r, k] * b[g * N + n, k]
                out[r, n] = s
    return out


def naive_wgrad(a_t, b_t, offs, G):
    N, M = a_t.shape
    K = b_t.shape[0]
    out = np.zeros((G, N, K))
    starts = [0] + list(offs[:-1])
    for g in range(G):
        for n in range(N):
            for k in range(K):
                s = 0.0
                for r in range(starts[g], offs[g]):
                    s += a_t[n, r] * b_t[k, r]
                out[g, n, k] = s
    return out


def test_grouped_mm_matches_loops(oracle):
    rng = np.random.default_rng(0)
    M, N, K, G = 12, 5, 7, 4
    offs = np.array([3, 3, 10, 12])  # group 1 is empty
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((G * N, K))
    got = oracle.grouped_mm(a, b, offs, G)
    assert np.allclose(got, naive_grouped(a, b, offs, G), rtol=1e-13, atol=1e-13)


def test_dense_is_one_group(oracle):
    rng = np.random.default_rng(1)
    a = rng.standard_normal((9, 6))
    b = rng.standard_normal((4, 6))
    got = oracle.grouped_mm(a, b, None, 1)
    assert np.allclose(got, naive_grouped(a, b, None, 1), rtol=1e-13, atol=1e-13)
    assert np.array_equal(got, oracle.grouped_mm(a, b, np.array([9]), 1))


def test_wgrad_matches_loops_and_empty_group_is_zero(oracle):
    rng = np.random.default_rng(2)
    N, K, M, G = 4, 5, 10, 3
    offs = np.array([4, 4, 10])
    a_t = rng.standard_normal((N, M))
    b_t = rng.standard_normal((K, M))
    got = oracle.grouped_mm_wgrad(a_t, b_t, offs, G)
    assert np.allclose(got, naive_wgrad(a_t, b_t, offs, G), rtol=1e-13, atol=1e-13)
    assert np.all(got[1] == 0)


def test_group_permutation_permutes_outputs(oracle):
    rng = np.random.default_rng(3)
    N, K, G = 3, 4, 3
    sizes = [2, 5, 3]
    a = rng.standard_normal((sum(sizes), K))
    b = rng.standard_normal((G * N, K))
    offs = np.cumsum(sizes)
    y = oracle.grouped_mm(a, b, offs, G)
    perm = [2, 0, 1]
    starts = np.concatenate([[0], offs[:-1]])
    a_p = np.concatenate([a[starts[g]:offs[g]] for g in perm])
    b_p = np.concatenate([b[g * N:(g + 1) * N] for g in perm])
    y_p = oracle.grouped_mm(a_p, b_p, np.cumsum([sizes[g] for g in perm]), G)
    assert np.array_equal(y_p, np.concatenate([y[starts[g]:offs[g]] for g in perm]))


def test_dgrad_is_forward_with_transposed_weight(oracle):
    """dX = dY W per group; the oracle takes W^T [G*K, N] as the second operand."""
    rng = np.random.default_rng(4)
    M, N, K, G = 8, 6, 5, 2
    offs = np.array([3, 8])
    dy = rng.standard_normal((M, N))
    w = rng.standard_normal((G, N, K))
    w_t = np.concatenate([w[g].T for g in range(G)])  # [G*K, N]
    dx = oracle.grouped_mm(dy, w_t, offs, G)
    for r in range(M):
        g = 0 if r < 3 else 1
        for k in range(K):
            assert math.isclose(dx[r, k], sum(dy[r, n] * w[g, n, k] for n in range(N)), rel_tol=1e-12, abs_tol=1e-12)


def test_exact_integer_case_matches_rationals(oracle):
    """Codes in {0, +-0.5, +-1, +-2} with scale bytes 126..128: every partial sum is exact."""
    rng = np.random.default_rng(5)
    M, N, K, G = 64, 32, 256, 2
    choices = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], np.uint8)
    a_q = rng.choice(choices, size=(M, K))
    b_q = rng.choice(choices, size=(G * N, K))
    a_s = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
    b_s = rng.integers(126, 129, size=(G * N, K // 32)).astype(np.uint8)
    offs = np.array([32, 64])
    got = oracle.mx_grouped_mm_fwd(a_q, a_s, b_q, b_s, offs, G)
    F = fractions.Fraction
    val = {0x00: F(0), 0x30: F(1, 2), 0xB0: F(-1, 2), 0x38: F(1), 0xB8: F(-1), 0x40: F(2), 0xC0: F(-2)}
    for r in range(0, M, 7):
        g = r // 32
        for n in range(0, N, 5):
            s = F(0)
            for k in range(K):
                sa = F(2) ** (int(a_s[r, k // 32]) - 127)
                sb = F(2) ** (int(b_s[g * N + n, k // 32]) - 127)
                s += val[int(a_q[r, k])] * sa * val[int(b_q[g * N + n, k])] * sb
            assert got[r, n] == float(s)


def exact_bf16_round(x):
    """Round-to-nearest-even to bf16 by exact rational arithmetic (normal range)."""
    F = fractions.Fraction
    fx = F(x)
    if fx == 0:
        return 0.0
    sign = -1 if fx < 0 else 1
    a = abs(fx)
    e = math.floor(math.log2(a))
    if F(2) ** e > a:
        e -= 1
    if F(2) ** (e + 1) <= a:
        e += 1
    q = F(2) ** (e - 7)
    n = a / q
    lo = math.floor(n)
    rem = n - lo
    if rem > F(1, 2) or (rem == F(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * float(lo * q)


def test_bf16_rounding(oracle):
    rng = np.random.default_rng(6)
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000))
    bits = oracle.round_to_bf16_bits(x)
    got = synth.bf16_bits_to_f32(bits).astype(np.float64)
    ref = np.array([exact_bf16_round(v) for v in x])
    assert np.array_equal(got, ref)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    t = oracle.round_to_bf16_bits(np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8)]))
    assert list(t) == [0x3F80, 0x3F82, 0xBF80]
    # a value that float32 would double-round: 1 + 2^-8 + 2^-30 must round up
    assert oracle.round_to_bf16_bits(np.array([1 + 2.0**-8 + 2.0**-30]))[0] == 0x3F81


def test_metrics(oracle):
    ref = np.array([3.0, 4.0])
    assert oracle.rel_frobenius(np.array([3.0, 4.5]), ref) == pytest.approx(0.1)
    assert oracle.sqnr_db(np.array([3.0, 4.5]), ref) == pytest.approx(10 * math.log10(25 / 0.25))
    o = oracle.bf16_ordinal(np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3F80], np.uint16))
    assert list(o) == [0, 0, 1, -1, 0x3F80]


def test_sqnr_small_linear(oracle):
    """The 256^3 MXFP8 linear against the unquantized bf16 product: >= 25 dB."""
    d = synth.linear_small(0)
    aq, as_ = oracle.quantize_dim0(d["a"])
    bq, bs = oracle.quantize_dim0(d["b"])
    y = oracle.mx_grouped_mm_fwd(aq, as_, bq, bs, None, 1)
    ref = oracle.bf16_to_f64(d["a"]) @ oracle.bf16_to_f64(d["b"]).T
    assert oracle.sqnr_db(y, ref) >= 25.0
