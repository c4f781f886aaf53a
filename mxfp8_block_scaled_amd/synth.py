"""Seeded synthetic inputs for the MXFP8 cast and grouped GEMM.

This module only draws inputs: bf16 bit patterns (uint16 arrays) and int32 group
offsets. It holds none of the MX arithmetic, so the tests can hand the very same
arrays to the HIP library and to the CPU oracle.

Recipe (shared by every workload):
  * one numpy Generator per tensor, spawned in a fixed order from
    SeedSequence(seed), so adding a tensor never changes the others;
  * "N(0, sigma)" means a normal with standard deviation sigma, drawn in float32,
    scaled, then rounded to bf16 with round-to-nearest-even; a tensor's rows are
    drawn in ~4M-element chunks, each from its own child of the tensor's generator;
  * group sizes are multiples of 32 rows (the grouped GEMM's alignment) and sum to
    the token count; offs holds their inclusive cumulative sums (group ends).

The workloads follow the shapes on the pages: the MXFP8Linear benchmark
(M=N=4096, K=2048; pytorch/ao PR 4705, linear benchmark command), the MoE
grouped-GEMM benchmark (K=N=4096, G=8, M=16384; same page, grouped benchmark
command), the 576-wide gradient (torchtitan PR 5334 body) and a DeepSeek-V3-like
one-GPU expert share (32 experts, hidden 7168, expert width 2048, top-8 routing).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even) and return uint16 bits.

    In uint32 arithmetic: a non-NaN pattern plus 0x7FFF plus its bit 16 stays below
    2^32 (the largest, -inf's 0xFF800000, gains at most 0x8000); NaNs map to 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u + np.uint32(0x7FFF)
    r += (u >> 16) & np.uint32(1)
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_CHUNK_ELEMS = 1 << 22
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def normal_bf16(rng, shape, std):
    """bf16 patterns of N(0, std) draws.

    The rows are cut into chunks of about 4M elements; chunk i draws from the i-th
    child generator spawned from `rng`, so the values depend only on the seed and
    the shape, and the chunks can be drawn on several threads (numpy releases the
    GIL while filling).
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1, shape[-1]) if len(shape) > 1 else out.reshape(1, -1)
    rows, cols = flat.shape
    chunk_rows = max(1, _CHUNK_ELEMS // max(cols, 1))
    starts = list(range(0, rows, chunk_rows))
    kids = rng.spawn(len(starts))

    def fill(i):
        r0 = starts[i]
        r1 = min(rows, r0 + chunk_rows)
        x = kids[i].standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= np.float32(std)
        flat[r0:r1] = f32_to_bf16_bits(x)

    if len(starts) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def spawn(seed, n):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def multinomial_groups(rng, total_rows, groups, align=32):
    """Equal-probability multinomial over `groups`, in units of `align` rows."""
    units = rng.multinomial(total_rows // align, [1.0 / groups] * groups)
    return (units * align).astype(np.int64)


def zipf_groups(rng, total_rows, groups, n_empty, exponent=1.2, align=32):
    """Zipf(exponent) group sizes with `n_empty` experts forced empty.

    The non-empty experts get probabilities proportional to rank^-exponent, the
    ranks assigned to experts by a seeded permutation; the row count is drawn
    multinomially in units of `align`. Should another expert come out empty by
    chance, one unit moves to it from the largest group, so exactly `n_empty`
    groups are empty.
    """
    perm = rng.permutation(groups)
    empty = set(perm[:n_empty].tolist())
    live = [g for g in perm[n_empty:].tolist()]
    p = np.arange(1, len(live) + 1, dtype=np.float64) ** (-exponent)
    p /= p.sum()
    units = np.zeros(groups, dtype=np.int64)
    units[live] = rng.multinomial(total_rows // align, p)
    for g in live:
        if units[g] == 0:
            units[int(np.argmax(units))] -= 1
            units[g] += 1
    assert all(units[g] == 0 for g in empty)
    return units * align


def offs_from_sizes(sizes):
    return np.cumsum(np.asarray(sizes, dtype=np.int64)).astype(np.int32)


# --------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------


def plant_blocks(rng, bits, frac=0.01, outlier=1e4):
    """Zero `frac` of the 1x32 row blocks and put one +-outlier in another `frac`.

    The two sets of blocks are disjoint. The outlier sits at a seeded position with
    a seeded sign; its value is bf16(1e4) = 9984.
    """
    R, C = bits.shape
    nblk = R * (C // 32)
    k = int(round(frac * nblk))
    pick = rng.choice(nblk, size=2 * k, replace=False)
    zero, spike = pick[:k], pick[k:]
    out = bits.copy().reshape(nblk, 32)
    out[zero] = 0
    pos = rng.integers(0, 32, size=k)
    sign = rng.integers(0, 2, size=k).astype(np.uint16)
    val = f32_to_bf16_bits(np.float32(outlier))
    out[spike, pos] = val | (sign << 15)
    return out.reshape(R, C)


def linear_small(seed=0):
    """Dense MXFP8 linear forward, 256x256x256 (the small parity workload).

    A ~ N(0,1), B ~ N(0,0.02), both [256, 256]; 1% of the 1x32 blocks of each zeroed
    and another 1% given a single +-9984 outlier.
    """
    r = spawn(seed, 4)
    a = plant_blocks(r[2], normal_bf16(r[0], (256, 256), 1.0))
    b = plant_blocks(r[3], normal_bf16(r[1], (256, 256), 0.02))
    return {"a": a, "b": b}


def linear_4096(seed=0):
    """Dense MXFP8Linear fwd+bwd: X [4096, 2048], W [4096, 2048], dY [4096, 4096]."""
    r = spawn(seed, 3)
    return {
        "x": normal_bf16(r[0], (4096, 2048), 1.0),
        "w": normal_bf16(r[1], (4096, 2048), 0.02),
        "dy": normal_bf16(r[2], (4096, 4096), 1e-2),
    }


def moe_g8(seed=0, with_backward=True, m=16384, k=4096, n=4096, groups=8, narrow=576):
    """MoE grouped GEMM: X [M, K], W [G, N, K], offs [G]; backward adds dY [M, N].

    With backward it also builds the unaligned dense layer: W' [576, K] and its
    gradient dY' [M, 576].
    """
    r = spawn(seed, 6)
    sizes = multinomial_groups(r[0], m, groups)
    d = {
        "offs": offs_from_sizes(sizes),
        "x": normal_bf16(r[1], (m, k), 1.0),
        "w": normal_bf16(r[2], (groups, n, k), 0.02),
    }
    if with_backward:
        d["dy"] = normal_bf16(r[3], (m, n), 1e-2)
        d["w_narrow"] = normal_bf16(r[4], (narrow, k), 0.02)
        d["dy_narrow"] = normal_bf16(r[5], (m, narrow), 1e-2)
    return d


def deepseek_share(seed=0, experts=32, hidden=7168, ffn=2048, tokens=4096, topk=8, scale_rows=1):
    """DeepSeek-V3-like expert share: 32 experts, hidden 7168, expert FFN 2048.

    Gate/up W1 [E, 2*ffn, hidden], down W2 [E, hidden, ffn]; X [T*topk, hidden]
    routed rows, H [T*topk, ffn] the down projection's input; gradients dY1
    [rows, 2*ffn], dY2 [rows, hidden]. Zipf(1.2) group sizes, 3 experts empty.
    `scale_rows` divides the row count for reduced-size variants.
    """
    rows = tokens * topk // scale_rows
    r = spawn(seed, 8)
    sizes = zipf_groups(r[0], rows, experts, n_empty=3)
    return {
        "offs": offs_from_sizes(sizes),
        "x": normal_bf16(r[1], (rows, hidden), 1.0),
        "w1": normal_bf16(r[2], (experts, 2 * ffn, hidden), 0.006),
        "w2": normal_bf16(r[3], (experts, hidden, ffn), 0.006),
        "h": normal_bf16(r[4], (rows, ffn), 1.0),
        "dy1": normal_bf16(r[5], (rows, 2 * ffn), 1e-2),
        "dy2": normal_bf16(r[6], (rows, hidden), 1e-2),
    }
