"""Pins for the oracle's physical scale layout.

The layout is fixed by what the gfx950 block-scaled MFMA (32x32x64, fp8) reads: the
scale for output row r and 32-wide k-block b of one 64-wide k-step comes from lane
r + 32*b of the scale register, and the instruction's byte selector picks one of
the register's four bytes. So one dword per lane serves four k-steps (eight
k-blocks) when lane l's dword holds the scales of row l%32 for k-blocks
l//32, 2 + l//32, 4 + l//32, 6 + l//32. These tests restate that requirement
with explicit loops and check the oracle's offset map against it.
"""

import itertools

import numpy as np
import pytest


@pytest.mark.parametrize("R,KB", [(32, 8), (64, 16), (33, 9), (576, 18), (1, 1), (100, 3)])
def test_layout_is_a_bijection_with_pads(oracle, R, KB):
    size = oracle.scale_bytes(R, KB)
    assert size == ((R + 31) // 32) * ((KB + 7) // 8) * 256
    r, kb = np.meshgrid(np.arange(R), np.arange(KB), indexing="ij")
    offs = oracle.scale_offset(r, kb, KB).ravel()
    assert offs.min() >= 0 and offs.max() < size
    assert len(np.unique(offs)) == R * KB
    rng = np.random.default_rng(R * 1000 + KB)
    logical = rng.integers(0, 255, size=(R, KB)).astype(np.uint8)
    phys = oracle.scales_to_physical(logical)
    assert phys.shape == (size,)
    mask = np.ones(size, bool)
    mask[offs] = False
    assert np.all(phys[mask] == 0x7F)
    assert np.array_equal(oracle.scales_from_physical(phys, R, KB), logical)


def test_layout_feeds_mfma_lanes(oracle):
    R, KB = 96, 24
    rng = np.random.default_rng(2)
    logical = rng.integers(0, 255, size=(R, KB)).astype(np.uint8)
    phys = oracle.scales_to_physical(logical)
    tiles_k = (KB + 7) // 8
    for rt, kt in itertools.product(range(R // 32), range(tiles_k)):
        base = (rt * tiles_k + kt) * 256
        for lane in range(64):
            for step in range(4):
                row = 32 * rt + lane % 32
                blk = 8 * kt + 2 * step + lane // 32
                assert phys[base + 4 * lane + step] == logical[row, blk]


def test_layout_tiles_run_along_k(oracle):
    """Consecutive 256-byte tiles of one row band cover consecutive groups of 8 k-blocks."""
    KB = 40
    for kt in range(5):
        assert oracle.scale_offset(0, 8 * kt, KB) == 256 * kt
        assert oracle.scale_offset(32, 8 * kt, KB) == 256 * (5 + kt)
