"""The instrumented build (libmxfp8_stamps.so, MX_CYCLE_STAMPS) behind bench.py
--cycle-stamps: its GEMMs give the product library's results bit for bit, and every
real tile leaves one record whose stamps are in order and whose k-steps are those of
its tile."""

import ctypes
import os

import numpy as np
import pytest

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import _lib, build, synth

from gpu_util import dev_bf16, dev_i32, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stamps():
    require_gpu()
    if not os.path.exists(build.STAMPS_LIB):
        pytest.skip("instrumented library not built (python -m mxfp8_block_scaled_amd.build --stamps)")
    lib = ctypes.CDLL(build.STAMPS_LIB)
    for name, (res, args) in _lib.SIGNATURES.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    lib.mx_cycle_stamps_blocks.restype = ctypes.c_int64
    lib.mx_cycle_stamps_read.argtypes = [ctypes.c_void_p]
    lib.mx_cycle_stamps_read.restype = ctypes.c_int
    lib.mx_cycle_stamps_clear.restype = ctypes.c_int
    return lib


def with_lib(lib, fn):
    """Runs fn with the binding calling `lib` (the product library otherwise)."""
    prev = _lib._lib
    _lib._lib = lib
    try:
        return fn()
    finally:
        _lib._lib = prev


def records(lib, fn):
    import torch

    torch.cuda.synchronize()
    assert lib.mx_cycle_stamps_clear() == 0
    out = with_lib(lib, fn)
    torch.cuda.synchronize()
    nb = lib.mx_cycle_stamps_blocks()
    buf = np.zeros(nb * 8, dtype=np.uint64)
    assert lib.mx_cycle_stamps_read(buf.ctypes.data) == 0
    rec = buf.reshape(nb, 8)
    return out, rec[rec[:, 7] == 1]


def check_order(rec):
    t0, t1, t2, t3 = (rec[:, i].astype(np.int64) for i in range(4))
    live = rec[:, 6] > 0
    assert np.all(t0[live] <= t1[live]) and np.all(t1[live] <= t2[live]) and np.all(t2[live] <= t3[live])
    assert np.all(t0 <= t3)


def test_grouped_fwd_records(stamps):
    m, n, k = 4096, 1024, 1024
    sizes = [1024, 0, 1536, 1536]  # one group empty
    offs = np.cumsum(sizes).astype(np.int32)
    rng = np.random.default_rng(7)
    xq, xs = mx.mx_quantize_dim0(dev_bf16(synth.normal_bf16(rng, (m, k), 1.0)))
    wq, ws = mx.mx_quantize_dim0(dev_bf16(synth.normal_bf16(rng, (len(sizes) * n, k), 0.02)))
    run = lambda: mx.mx_grouped_mm_fwd(xq, xs, wq, ws, dev_i32(offs), m, n, k)  # noqa: E731
    ref = host(run())
    got, rec = records(stamps, run)
    assert np.array_equal(host(got), ref)
    # 128x128 tiles at this size: one record per real tile, k / 64 steps each
    tiles = sum((s + 127) // 128 for s in sizes) * (n // 128)
    say(f"fwd: {len(rec)} records for {tiles} tiles")
    assert len(rec) == tiles
    assert np.all(rec[:, 6] == k // 64)
    check_order(rec)


def test_grouped_wgrad_records(stamps):
    m, n, k = 4096, 512, 512
    sizes = [1056, 0, 32, 3008]  # an empty group, a one-block group, edges off the 256 grid
    offs = np.cumsum(sizes).astype(np.int32)
    rng = np.random.default_rng(8)
    _, _, dytq, dyts = mx.mx_quantize_dim0_dim1(dev_bf16(synth.normal_bf16(rng, (m, n), 1e-2)))
    _, _, xtq, xts = mx.mx_quantize_dim0_dim1(dev_bf16(synth.normal_bf16(rng, (m, k), 1.0)))
    # unsplit (no workspace): one record per output tile and group
    run = lambda: mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, dev_i32(offs), m, n, k, workspace=None)  # noqa: E731
    ref = host(run())
    got, rec = records(stamps, run)
    assert np.array_equal(host(got), ref)
    # every group's tiles are launched, empty groups included (they write zeros); a
    # tile's loop starts at the 256-aligned position at or below its group's start
    starts = np.concatenate([[0], offs[:-1]])
    steps = [(-(-(e - s // 256 * 256) // 64)) if e > s else 0 for s, e in zip(starts, offs)]
    per_group = len(rec) // len(sizes)
    assert len(rec) == per_group * len(sizes) and per_group >= 1
    want = np.sort(np.repeat(steps, per_group))
    say(f"wgrad: {len(rec)} records, k-steps per group {steps}")
    assert np.array_equal(np.sort(rec[:, 6].astype(np.int64)), want)
    check_order(rec)
