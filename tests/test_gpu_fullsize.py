"""GEMM parity at full workload sizes, on sampled outputs.

Two workloads run through the same calls the benchmark makes (the one-pass dim0 +
dim1 cast of every tensor, the 32x32 cast of the narrow weight, then the grouped
GEMMs):
  * the MoE grouped GEMM (G=8 experts, 16384 tokens, K=N=4096; multinomial group
    sizes) with its fwd, dgrad and wgrad, all bf16 out, and the 576-wide dense
    layer beside it (32x32 weight scales; dgrad contracts over 576, the padded
    path);
  * the DeepSeek-V3-like one-GPU expert share (32 experts, 32768 routed rows with
    Zipf(1.2) group sizes and three empty experts, hidden 7168, expert width
    2048): gate/up (N=4096, K=7168) and down (N=7168, K=2048), each fwd, dgrad
    and wgrad.
The oracle recomputes sampled outputs one by one. dim0 scales belong to one row
and dim1 scales to one column, so quantizing only the sampled rows of one operand
and the sampled rows or columns of the other gives exactly the codes the full
casts give there. Samples: every non-empty group's first and last row plus
random rows; the first and last column, both sides of a 256-column tile boundary
and random columns. Every empty expert's wgrad is checked to be all zeros. Each sampled
output is held to the block-scaled MFMA model's tolerance (tests/mfma_model.py) and
to the model's worst-case bound of the exact value (gemm_check.check_mx).
"""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import synth

import mfma_model
from gemm_check import check_mx, check_mx_wgrad
from gpu_util import dev_bf16, dev_i32, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def group_ranges(offs):
    ends = [int(o) for o in offs]
    return list(zip([0] + ends[:-1], ends))


def pick(rng, lo, hi, n):
    """Sorted distinct indices in [lo, hi): both ends plus n random ones."""
    if hi <= lo:
        return np.zeros(0, np.int64)
    return np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, size=n)])).astype(np.int64)


def pick_cols(rng, n, count):
    fixed = [0, n - 1] + ([255, 256] if n > 256 else [])
    return np.unique(np.concatenate([fixed, rng.integers(0, n, size=count)])).astype(np.int64)


def gather(t, rows, cols):
    r = torch.from_numpy(rows).to(t.device)
    c = torch.from_numpy(cols).to(t.device)
    return host(t.index_select(0, r).index_select(1, c).contiguous())


def check_rows(oracle, name, got_dev, a_bits, rows_by_group, cols, b_rows, K, out_bf16=True):
    """Y[r, c] for r in the sampled rows of each group, c in cols, against the oracle and
    the MFMA model.

    a_bits: the dim0-cast operand's bf16 bits [M, K]; b_rows(g) gives the oracle's
    (codes, logical scales) of the other operand's rows `cols` for group g.
    """
    refs, hs, abs_, bounds, rows = [], [], [], [], []
    for g, R in rows_by_group:
        oa, oas = oracle.quantize_dim0(a_bits[R])
        ob, obs = b_rows(g)
        refs.append(oracle.dequantize(oa, oas) @ oracle.dequantize(ob, obs).T)
        h, ab = mfma_model.run_truncated_mm(oa, oas, ob, obs)
        hs.append(h)
        abs_.append(ab)
        bounds.append(mfma_model.run_bound_mm(oa, oas, ob, obs))
        rows.append(R)
    rows = np.concatenate(rows)
    got = gather(got_dev, rows, cols)
    say(f"    {name}: {got.size} sampled outputs over {len(rows_by_group)} groups")
    check_mx(oracle, got, np.concatenate(refs), np.concatenate(abs_), K, name, h=np.concatenate(hs),
             bound=np.concatenate(bounds), out_bf16=out_bf16)


def check_wgrad(oracle, name, dw_dev, dy_bits, x_bits, offs, cols_n, cols_k, out_bf16):
    G = len(offs)
    odyt, odyts = oracle.quantize_dim1(dy_bits[:, cols_n])
    oxt, oxts = oracle.quantize_dim1(x_bits[:, cols_k])
    n = torch.from_numpy(cols_n).to(dw_dev.device)
    k = torch.from_numpy(cols_k).to(dw_dev.device)
    got = host(dw_dev.index_select(1, n).index_select(2, k).contiguous())
    live = [g for g, (s, e) in enumerate(group_ranges(offs)) if e > s]
    say(f"    {name}: {got[live].size} sampled outputs over {len(live)} groups")
    check_mx_wgrad(oracle, got, odyt, odyts, oxt, oxts, offs, G, name, out_bf16=out_bf16)
    for g, (s, e) in enumerate(group_ranges(offs)):
        if e == s:
            assert int(torch.count_nonzero(dw_dev[g])) == 0, f"{name}: empty group {g} has nonzero wgrad"


# ---------------------------------------------------------------------------------------
# MoE grouped GEMM, G=8, M=16384, K=N=4096, and the 576-wide dense layer
# ---------------------------------------------------------------------------------------


@pytest.fixture(scope="module")
def moe():
    say("[full-size moe_g8] generating")
    d = synth.moe_g8(0, with_backward=True)
    dev = {k: dev_bf16(v) for k, v in d.items() if k != "offs"}
    dev["offs"] = dev_i32(d["offs"])
    say("[full-size moe_g8] one-pass casts of X, W (8 x 4096 x 4096), dY, dY'")
    for name in ("x", "w", "dy", "dy_narrow"):
        dev[name + "_q"] = mx.mx_quantize_dim0_dim1(dev[name])  # (q, scale, q_t, scale_t)
    return d, dev


def test_moe_g8_fwd(oracle, moe):
    d, t = moe
    M, K = d["x"].shape
    G, N, _ = d["w"].shape
    xq, xs = t["x_q"][:2]
    wq, ws = t["w_q"][:2]
    y = mx.mx_grouped_mm_fwd(xq, xs, wq, ws, t["offs"], M, N, K)
    rng = np.random.default_rng(1)
    rows = [(g, pick(rng, s, e, 6)) for g, (s, e) in enumerate(group_ranges(d["offs"])) if e > s]
    cols = pick_cols(rng, N, 20)
    check_rows(oracle, "moe fwd bf16", y, d["x"], rows, cols, lambda g: oracle.quantize_dim0(d["w"][g][cols]), K)


def test_moe_g8_dgrad(oracle, moe):
    d, t = moe
    M, K = d["x"].shape
    G, N, _ = d["w"].shape
    dyq, dys = t["dy_q"][:2]
    wtq, wts = t["w_q"][2:]
    dx = mx.mx_grouped_mm_dgrad(dyq, dys, wtq, wts, t["offs"], M, N, K)
    rng = np.random.default_rng(2)
    rows = [(g, pick(rng, s, e, 6)) for g, (s, e) in enumerate(group_ranges(d["offs"])) if e > s]
    cols = pick_cols(rng, K, 20)
    check_rows(oracle, "moe dgrad bf16", dx, d["dy"], rows, cols,
               lambda g: oracle.quantize_dim1(d["w"][g][:, cols]), N)


def test_moe_g8_wgrad(oracle, moe):
    d, t = moe
    M, K = d["x"].shape
    G, N, _ = d["w"].shape
    dytq, dyts = t["dy_q"][2:]
    xtq, xts = t["x_q"][2:]
    dw = mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, t["offs"], M, N, K, out_dtype=mx.MX_OUT_BF16)
    rng = np.random.default_rng(3)
    check_wgrad(oracle, "moe wgrad bf16", dw, d["dy"], d["x"], d["offs"], pick_cols(rng, N, 16),
                pick_cols(rng, K, 16), True)


def test_dense576_fwd_dgrad_wgrad(oracle, moe):
    d, t = moe
    M, K = d["x"].shape
    Nn = d["w_narrow"].shape[0]
    owq, owqt, owsr, owsc = oracle.quantize_weight_32x32(d["w_narrow"])
    wq, wqt, wsr, wsc = mx.mx_quantize_weight_32x32(t["w_narrow"])
    xq, xs = t["x_q"][:2]
    rng = np.random.default_rng(4)
    rows = [(0, pick(rng, 0, M, 40))]
    y = mx.mx_grouped_mm_fwd(xq, xs, wq, wsr, None, M, Nn, K)
    cols = pick_cols(rng, Nn, 20)
    check_rows(oracle, "dense576 fwd bf16", y, d["x"], rows, cols, lambda g: (owq[cols], owsr[cols]), K)
    dyq, dys = t["dy_narrow_q"][:2]
    dx = mx.mx_grouped_mm_dgrad(dyq, dys, wqt, wsc, None, M, Nn, K)
    cols = pick_cols(rng, K, 20)
    check_rows(oracle, "dense576 dgrad bf16 (contraction 576)", dx, d["dy_narrow"], rows, cols,
               lambda g: (owqt[cols], owsc[cols]), Nn)
    dytq, dyts = t["dy_narrow_q"][2:]
    xtq, xts = t["x_q"][2:]
    dw = mx.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, None, M, Nn, K, out_dtype=mx.MX_OUT_BF16)
    check_wgrad(oracle, "dense576 wgrad bf16", dw, d["dy_narrow"], d["x"], np.array([M], np.int32),
                pick_cols(rng, Nn, 16), pick_cols(rng, K, 16), True)


# ---------------------------------------------------------------------------------------
# DeepSeek-V3-like expert share: 32 experts, Zipf group sizes with three empty experts
# ---------------------------------------------------------------------------------------


@pytest.fixture(scope="module")
def share():
    say("[full-size deepseek share] generating")
    d = synth.deepseek_share(0)
    dev = {k: dev_bf16(v) for k, v in d.items() if k != "offs"}
    dev["offs"] = dev_i32(d["offs"])
    sizes = np.diff(np.concatenate([[0], d["offs"]]))
    say(f"    group sizes: {sizes.tolist()}")
    assert np.sum(sizes == 0) == 3
    return d, dev


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_share_fwd_dgrad(oracle, share, proj):
    d, t = share
    a, w, dy = ("x", "w1", "dy1") if proj == "gate_up" else ("h", "w2", "dy2")
    M, K = d[a].shape
    G, N, _ = d[w].shape
    rng = np.random.default_rng(5 if proj == "gate_up" else 6)
    rows = [(g, pick(rng, s, e, 3)) for g, (s, e) in enumerate(group_ranges(d["offs"])) if e > s]
    aq, as_, _, _ = mx.mx_quantize_dim0_dim1(t[a])
    wq, ws, wtq, wts = mx.mx_quantize_dim0_dim1(t[w])
    y = mx.mx_grouped_mm_fwd(aq, as_, wq, ws, t["offs"], M, N, K)
    cols = pick_cols(rng, N, 12)
    check_rows(oracle, f"share {proj} fwd bf16", y, d[a], rows, cols,
               lambda g: oracle.quantize_dim0(d[w][g][cols]), K)
    del aq, as_, wq, ws, y
    dyq, dys, _, _ = mx.mx_quantize_dim0_dim1(t[dy])
    dx = mx.mx_grouped_mm_dgrad(dyq, dys, wtq, wts, t["offs"], M, N, K)
    cols = pick_cols(rng, K, 12)
    check_rows(oracle, f"share {proj} dgrad bf16", dx, d[dy], rows, cols,
               lambda g: oracle.quantize_dim1(d[w][g][:, cols]), N)


@pytest.mark.parametrize("proj,out_dtype", [("gate_up", mx.MX_OUT_F32), ("down", mx.MX_OUT_BF16)])
def test_share_wgrad(oracle, share, proj, out_dtype):
    d, t = share
    a, w, dy = ("x", "w1", "dy1") if proj == "gate_up" else ("h", "w2", "dy2")
    M, K = d[a].shape
    G, N, _ = d[w].shape
    _, _, dytq, dyts = mx.mx_quantize_dim0_dim1(t[dy])
    _, _, atq, ats = mx.mx_quantize_dim0_dim1(t[a])
    dw = mx.mx_grouped_mm_wgrad(dytq, dyts, atq, ats, t["offs"], M, N, K, out_dtype=out_dtype)
    rng = np.random.default_rng(7 if proj == "gate_up" else 8)
    check_wgrad(oracle, f"share {proj} wgrad {'bf16' if out_dtype else 'f32'}", dw, d[dy], d[a], d["offs"],
                pick_cols(rng, N, 12), pick_cols(rng, K, 12), out_dtype == mx.MX_OUT_BF16)
