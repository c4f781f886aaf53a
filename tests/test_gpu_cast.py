"""GPU parity of the three MXFP8 casts against the CPU oracle: codes and scales
must be bit-exact, and the physical scale buffer byte-for-byte (pads included)."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import synth

from gpu_util import dev_bf16, host, require_gpu, say, stress_blocks

pytestmark = pytest.mark.gpu


def check_dim0(oracle, bits, name):
    say(f"[cast dim0] {name} shape={bits.shape}")
    q, s = mx.mx_quantize_dim0(dev_bf16(bits))
    oq, osl = oracle.quantize_dim0(bits)
    gq = host(q)
    assert np.array_equal(gq, oq), f"{name}: {np.sum(gq != oq)} code mismatches"
    gs = host(s)
    assert np.array_equal(gs, oracle.scales_to_physical(osl)), name


def check_dim1(oracle, bits, name):
    say(f"[cast dim1] {name} shape={bits.shape}")
    q_t, s_t = mx.mx_quantize_dim1(dev_bf16(bits))
    gq = host(q_t)
    if bits.ndim == 2:
        oq, osl = oracle.quantize_dim1(bits)
    else:
        parts = [oracle.quantize_dim1(b) for b in bits]
        oq = np.stack([p[0] for p in parts])
        osl = np.concatenate([p[1] for p in parts])
    assert np.array_equal(gq, oq), f"{name}: {np.sum(gq != oq)} code mismatches"
    assert np.array_equal(host(s_t), oracle.scales_to_physical(osl)), name


def check_w32(oracle, bits, name):
    say(f"[cast w32] {name} shape={bits.shape}")
    q, q_t, s_row, s_col = mx.mx_quantize_weight_32x32(dev_bf16(bits))
    if bits.ndim == 2:
        oq, oqt, osr, osc = oracle.quantize_weight_32x32(bits)
    else:
        parts = [oracle.quantize_weight_32x32(b) for b in bits]
        oq = np.stack([p[0] for p in parts])
        oqt = np.stack([p[1] for p in parts])
        osr = np.concatenate([p[2] for p in parts])
        osc = np.concatenate([p[3] for p in parts])
    assert np.array_equal(host(q), oq), name
    assert np.array_equal(host(q_t), oqt), name
    assert np.array_equal(host(s_row), oracle.scales_to_physical(osr)), name
    assert np.array_equal(host(s_col), oracle.scales_to_physical(osc)), name


def check_both(oracle, bits, name, stream_t=False):
    """The one-pass cast must equal dim0 of the stacked rows and dim1, bit for bit
    (stream_t: q_t written with non-temporal stores, same values)."""
    say(f"[cast dim0+dim1] {name} shape={bits.shape} stream_t={stream_t}")
    q, s, q_t, s_t = mx.mx_quantize_dim0_dim1(dev_bf16(bits), stream_t=stream_t)
    stacked = bits.reshape(-1, bits.shape[-1])
    oq, osl = oracle.quantize_dim0(stacked)
    gq = host(q)
    assert np.array_equal(gq, oq), f"{name}: {np.sum(gq != oq)} dim0 code mismatches"
    assert np.array_equal(host(s), oracle.scales_to_physical(osl)), name
    if bits.ndim == 2:
        oqt, ost = oracle.quantize_dim1(bits)
    else:
        parts = [oracle.quantize_dim1(b) for b in bits]
        oqt = np.stack([p[0] for p in parts])
        ost = np.concatenate([p[1] for p in parts])
    gqt = host(q_t)
    assert np.array_equal(gqt, oqt), f"{name}: {np.sum(gqt != oqt)} dim1 code mismatches"
    assert np.array_equal(host(s_t), oracle.scales_to_physical(ost)), name


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


@pytest.mark.parametrize("shape", [(1, 32), (37, 96), (64, 256), (33, 288), (100, 576), (257, 1056)])
def test_dim0_shapes(oracle, shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    check_dim0(oracle, synth.normal_bf16(rng, shape, 1.0), f"normal{shape}")


def test_dim0_stress_every_amax(oracle):
    blocks = stress_blocks(0)
    n = blocks.shape[0] // 8 * 8
    check_dim0(oracle, blocks[:n].reshape(-1, 256), "stress")
    check_dim0(oracle, blocks[n:].reshape(-1, 32), "stress-tail")


def test_dim0_small_linear_inputs(oracle):
    d = synth.linear_small(0)
    check_dim0(oracle, d["a"], "A 256x256 with zero/outlier blocks")
    check_dim0(oracle, d["b"], "B 256x256 with zero/outlier blocks")


def test_dim0_strided_input(oracle):
    rng = np.random.default_rng(9)
    big = synth.normal_bf16(rng, (64, 320), 1.0)
    x = dev_bf16(big)[:, 32:288]  # row pitch 320, 256 columns
    q, s = mx.mx_quantize_dim0(x)
    oq, osl = oracle.quantize_dim0(big[:, 32:288])
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(s), oracle.scales_to_physical(osl))


def test_dim0_full_size_sampled_rows(oracle):
    """16384x4096 tokens: every byte checked against the oracle on 1024 sampled rows."""
    d = synth.moe_g8(0, with_backward=False)
    x = d["x"]
    say("[cast dim0] 16384x4096 sampled")
    q, s = mx.mx_quantize_dim0(dev_bf16(x))
    gq, gs = host(q), host(s)
    rows = np.sort(np.random.default_rng(1).choice(x.shape[0], 1024, replace=False))
    oq, osl = oracle.quantize_dim0(x[rows])
    assert np.array_equal(gq[rows], oq)
    assert np.array_equal(oracle.scales_from_physical(gs, x.shape[0], x.shape[1] // 32)[rows], osl)


@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (96, 160), (288, 64), (256, 576), (544, 1056)])
def test_dim1_shapes(oracle, shape):
    rng = np.random.default_rng(shape[0] * 3 + shape[1])
    check_dim1(oracle, synth.normal_bf16(rng, shape, 1.0), f"normal{shape}")


def test_dim1_stress_every_amax(oracle):
    blocks = stress_blocks(1)
    n = blocks.shape[0] // 64 * 64
    # blocks become columns: column c of a [32, 64] panel is block c
    panels = blocks[:n].reshape(-1, 64, 32).transpose(0, 2, 1).reshape(-1, 64)
    check_dim1(oracle, np.ascontiguousarray(panels), "stress")


def test_dim1_batched(oracle):
    rng = np.random.default_rng(5)
    check_dim1(oracle, synth.normal_bf16(rng, (3, 64, 96), 0.02), "batch3")


def test_dim1_full_size_sampled_columns(oracle):
    d = synth.moe_g8(0, with_backward=False)
    x = d["x"]
    say("[cast dim1] 16384x4096 sampled")
    q_t, s_t = mx.mx_quantize_dim1(dev_bf16(x))
    gq, gs = host(q_t), host(s_t)
    cols = np.sort(np.random.default_rng(2).choice(x.shape[1], 128, replace=False))
    oq, osl = oracle.quantize_dim0(np.ascontiguousarray(x[:, cols].T))
    assert np.array_equal(gq[cols], oq)
    assert np.array_equal(oracle.scales_from_physical(gs, x.shape[1], x.shape[0] // 32)[cols], osl)


@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (96, 160), (288, 64), (256, 576), (544, 1056), (512, 768)])
def test_dim0_dim1_shapes(oracle, shape):
    rng = np.random.default_rng(shape[0] * 5 + shape[1])
    check_both(oracle, synth.normal_bf16(rng, shape, 1.0), f"normal{shape}")


def test_dim0_dim1_stress_every_amax(oracle):
    """Every bf16 amax as a row block and, from transposed panels, as a column block."""
    blocks = stress_blocks(2)
    n_row = blocks.shape[0] // 256 * 256  # 8 blocks per 256-column row, rows a multiple of 32
    check_both(oracle, np.ascontiguousarray(blocks[:n_row].reshape(-1, 256)), "row blocks")
    n_col = blocks.shape[0] // 64 * 64
    panels = blocks[:n_col].reshape(-1, 64, 32).transpose(0, 2, 1).reshape(-1, 64)  # column c of a panel = block c
    check_both(oracle, np.ascontiguousarray(panels), "column blocks")


def test_dim0_dim1_batched(oracle):
    rng = np.random.default_rng(6)
    check_both(oracle, synth.normal_bf16(rng, (3, 96, 320), 0.02), "batch3")


def test_dim0_dim1_four_wave_path(oracle):
    """More tiles than compute units (17 x 17 tiles of 256 x 256, the last column tile
    partial): the four-wave workgroups, which small shapes never reach; full outputs,
    and batched: 5 x 5 x 13 tiles with a partial row tile per batch."""
    rng = np.random.default_rng(7)
    check_both(oracle, synth.normal_bf16(rng, (4352, 4160), 1.0), "2D 289 tiles")
    check_both(oracle, synth.normal_bf16(rng, (5, 1056, 3328), 0.02), "batch5 325 tiles")


@pytest.mark.parametrize("stream_t", [False, True])
def test_dim0_dim1_stream_hint(oracle, stream_t):
    """MX_FORM_STREAM_T changes only where q_t is cached: both paths bit-exact, on the
    eight- and four-wave workgroups, 2D and batched."""
    rng = np.random.default_rng(11)
    check_both(oracle, synth.normal_bf16(rng, (300, 576), 1.0)[:288], "2D eight-wave", stream_t)
    check_both(oracle, synth.normal_bf16(rng, (3, 2080, 1056), 0.02), "batch3 four-wave", stream_t)


def test_dim0_dim1_full_size_sampled(oracle):
    d = synth.moe_g8(0, with_backward=False)
    x = d["x"]
    say("[cast dim0+dim1] 16384x4096 sampled")
    q, s, q_t, s_t = mx.mx_quantize_dim0_dim1(dev_bf16(x))
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(x.shape[0], 128, replace=False))
    cols = np.sort(rng.choice(x.shape[1], 128, replace=False))
    oq, osl = oracle.quantize_dim0(x[rows])
    assert np.array_equal(host(q)[rows], oq)
    assert np.array_equal(oracle.scales_from_physical(host(s), x.shape[0], x.shape[1] // 32)[rows], osl)
    oqt, ost = oracle.quantize_dim0(np.ascontiguousarray(x[:, cols].T))
    assert np.array_equal(host(q_t)[cols], oqt)
    assert np.array_equal(oracle.scales_from_physical(host(s_t), x.shape[1], x.shape[0] // 32)[cols], ost)


@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (96, 288), (576, 512)])
def test_w32_shapes(oracle, shape):
    rng = np.random.default_rng(shape[0] + shape[1])
    check_w32(oracle, synth.normal_bf16(rng, shape, 0.02), f"normal{shape}")


def test_w32_zero_and_tiny_tiles(oracle):
    rng = np.random.default_rng(8)
    w = synth.normal_bf16(rng, (64, 64), 0.02)
    w[:32, :32] = 0
    w[32:, :32] = np.where(rng.random((32, 32)) < 0.5, 0x0003, 0x8001)  # denormal tile
    check_w32(oracle, w, "zero and denormal tiles")


def test_w32_batched(oracle):
    rng = np.random.default_rng(10)
    check_w32(oracle, synth.normal_bf16(rng, (2, 64, 96), 0.02), "batch2")


def test_w32_linear_weight(oracle):
    d = synth.linear_4096(0)
    check_w32(oracle, d["w"], "W 4096x2048")


def test_casts_deterministic():
    rng = np.random.default_rng(11)
    x = dev_bf16(synth.normal_bf16(rng, (512, 1024), 1.0))
    a = [host(t) for t in mx.mx_quantize_dim1(x)]
    b = [host(t) for t in mx.mx_quantize_dim1(x)]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def oracle_forms(oracle, bits, mode):
    stacked = bits.reshape(-1, bits.shape[-1])
    oq, osl = oracle.quantize_dim0(stacked, mode)
    if bits.ndim == 2:
        oqt, ost = oracle.quantize_dim1(bits, mode)
    else:
        parts = [oracle.quantize_dim1(b, mode) for b in bits]
        oqt = np.stack([p[0] for p in parts])
        ost = np.concatenate([p[1] for p in parts])
    return oq, oracle.scales_to_physical(osl), oqt, oracle.scales_to_physical(ost)


def check_ex(oracle, bits, forms, mode, name):
    say(f"[cast ex] {name} forms={forms} mode={mode} shape={bits.shape}")
    q, s, q_t, s_t = mx.mx_quantize_ex(dev_bf16(bits), forms, mode)
    oq, os_, oqt, ost = oracle_forms(oracle, bits, "floor" if mode == mx.MX_SCALE_FLOOR else "rceil")
    if forms & mx.MX_FORM_DIM0:
        gq = host(q)
        assert np.array_equal(gq, oq), f"{name}: {np.sum(gq != oq)} dim0 code mismatches"
        assert np.array_equal(host(s), os_), name
    else:
        assert q is None and s is None
    if forms & mx.MX_FORM_DIM1:
        gqt = host(q_t)
        assert np.array_equal(gqt, oqt), f"{name}: {np.sum(gqt != oqt)} dim1 code mismatches"
        assert np.array_equal(host(s_t), ost), name
    else:
        assert q_t is None and s_t is None


@pytest.mark.parametrize("forms", [1, 2, 3])
@pytest.mark.parametrize("shape", [(64, 96), (288, 576), (3, 96, 320)])
def test_floor_forms(oracle, forms, shape):
    rng = np.random.default_rng(sum(shape) + forms)
    check_ex(oracle, synth.normal_bf16(rng, shape, 1.0), forms, mx.MX_SCALE_FLOOR, f"normal{shape}")


def test_floor_four_wave_path(oracle):
    """FLOOR through the four-wave one-pass workgroups (17 x 17 tiles)."""
    rng = np.random.default_rng(8)
    check_ex(oracle, synth.normal_bf16(rng, (4352, 4160), 1.0), 3, mx.MX_SCALE_FLOOR, "2D 289 tiles")


def test_floor_stress_every_amax(oracle):
    blocks = stress_blocks(3)
    n_row = blocks.shape[0] // 256 * 256
    check_ex(oracle, np.ascontiguousarray(blocks[:n_row].reshape(-1, 256)), 3, mx.MX_SCALE_FLOOR, "row blocks")
    n_col = blocks.shape[0] // 64 * 64
    panels = blocks[:n_col].reshape(-1, 64, 32).transpose(0, 2, 1).reshape(-1, 64)
    check_ex(oracle, np.ascontiguousarray(panels), 3, mx.MX_SCALE_FLOOR, "column blocks")
    check_ex(oracle, np.ascontiguousarray(panels), 2, mx.MX_SCALE_FLOOR, "column blocks, dim1 kernel")
    check_ex(oracle, np.ascontiguousarray(blocks[:n_row].reshape(-1, 256)), 1, mx.MX_SCALE_FLOOR, "rows, dim0 kernel")


def test_ex_rceil_matches_plain_entry_points():
    rng = np.random.default_rng(9)
    x = dev_bf16(synth.normal_bf16(rng, (2, 160, 288), 1.0))
    q, s, q_t, s_t = mx.mx_quantize_ex(x, 3, mx.MX_SCALE_RCEIL)
    q0, s0 = mx.mx_quantize_dim0(x.view(-1, 288))
    q1, s1 = mx.mx_quantize_dim1(x)
    for a, b in ((q, q0), (s, s0), (q_t, q1), (s_t, s1)):
        assert torch.equal(a, b)
