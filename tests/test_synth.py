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
