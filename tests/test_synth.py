"""Checks of the seeded input generators (shapes, alignment, determinism)."""

import numpy as np

from mxfp8_block_scaled_amd import synth


def test_bf16_rounding_of_inputs():
    x = np.array([1.0, 1 + 2.0**-8, 1 + 3 * 2.0**-8, -2.5, 0.0], np.float32)
    assert list(synth.f32_to_bf16_bits(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000]


def test_multinomial_groups():
    rng = np.random.default_rng(0)
    s = synth.multinomial_groups(rng, 16384, 8)
    assert s.sum() == 16384 and np.all(s % 32 == 0) and len(s) == 8


def test_zipf_groups_three_empty():
    for seed in range(5):
        rng = np.random.default_rng(seed)
        s = synth.zipf_groups(rng, 32768, 32, n_empty=3)
        assert s.sum() == 32768 and np.all(s % 32 == 0)
        assert np.sum(s == 0) == 3


def test_linear_small_planted_blocks():
    d = synth.linear_small(0)
    for name in ("a", "b"):
        blk = d[name].reshape(-1, 32)
        assert np.sum(np.all(blk == 0, axis=1)) >= 20
        assert np.sum(np.any((blk & 0x7FFF) == 0x461C, axis=1)) == 20
    assert np.array_equal(synth.linear_small(0)["a"], d["a"])


def test_moe_offsets():
    d = synth.moe_g8(0, with_backward=False, m=1024, k=64, n=64)
    assert d["offs"][-1] == 1024 and np.all(np.diff(np.concatenate([[0], d["offs"]])) >= 0)
    assert d["offs"].dtype == np.int32


def test_bf16_rounding_matches_nearest_even_in_float64():
    """The uint32 rounding picks the nearer of the two bf16 neighbours, ties to the even one."""
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, np.array([0x3F808000, 0x3F818000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00008000, 0x80018000],
                                    np.uint32)])
    x = u.view(np.float32)
    keep = np.isfinite(x)
    u, x = u[keep], x[keep]
    lo = (u >> 16).astype(np.uint32)  # truncation toward zero in magnitude
    hi = lo + 1
    as64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    xv = x.astype(np.float64)
    dlo, dhi = np.abs(xv - as64(lo)), np.abs(as64(hi) - xv)
    hi_inf = (hi & 0x7FFF) == 0x7F80
    dhi = np.where(hi_inf, np.abs(np.ldexp(1.0, 128) * np.sign(xv) - xv), dhi)  # overflow rounds as 2^128
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi))).astype(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), want)


def test_normal_bf16_independent_of_thread_count(monkeypatch):
    def draw():
        return synth.normal_bf16(np.random.default_rng(11), (3000, 2048), 0.5)  # two chunks

    a = draw()
    monkeypatch.setattr(synth, "_THREADS", 1)
    b = draw()
    assert np.array_equal(a, b)
    v = synth.bf16_bits_to_f32(a).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 0.5) < 0.01
