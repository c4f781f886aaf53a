"""offs on the device: mx_check_offs reports every kind of violation, and the grouped
GEMMs stay inside their buffers when offs breaks the preconditions.

The memory-safety cases pass the operand and the output as views into buffers with
256 guard rows on each side and break offs by at most 64 rows, so every access of
the call, right or wrong, stays inside memory this test owns; the guard rows must
come back untouched. The forward must then equal the oracle on the offs the kernel
reads: the running maximum of the ends clamped into [0, m].
"""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import synth

from gpu_util import dev_i32, dev_u8, host, require_gpu, say

pytestmark = pytest.mark.gpu

GUARD = 256


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


@pytest.mark.parametrize("offs,m,multiple,bits,first", [
    ([32, 64, 64, 128], 128, 32, 0, -1),
    ([32, 64, 32, 128], 128, 32, mx.MX_OFFS_DECREASING, 2),
    ([32, 70, 96, 128], 128, 32, mx.MX_OFFS_NOT_MULTIPLE, 1),
    ([32, 70, 96, 128], 128, 1, 0, -1),
    ([32, 64, 96, 160], 128, 32, mx.MX_OFFS_OUT_OF_RANGE, 3),
    ([-32, 64, 96, 128], 128, 32, mx.MX_OFFS_DECREASING | mx.MX_OFFS_OUT_OF_RANGE, 0),
    ([96, 64, 100, 200], 128, 32,
     mx.MX_OFFS_DECREASING | mx.MX_OFFS_NOT_MULTIPLE | mx.MX_OFFS_OUT_OF_RANGE, 1),
])
def test_check_offs_flags(offs, m, multiple, bits, first):
    say(f"[check offs] {offs} m={m} multiple={multiple}")
    res = host(mx.mx_check_offs(dev_i32(np.array(offs, np.int32)), m, multiple)).tolist()
    assert res == [bits, first]


def test_check_offs_many_groups():
    """3000 groups, the first violation far from the start (several threads' ranges)."""
    offs = np.arange(1, 3001, dtype=np.int32) * 32
    offs[2500] = offs[2499] - 32  # decreasing
    offs[2700] += 1  # not a multiple
    res = host(mx.mx_check_offs(dev_i32(offs), int(offs.max()), 32)).tolist()
    assert res == [mx.MX_OFFS_DECREASING | mx.MX_OFFS_NOT_MULTIPLE, 2500]
    good = np.arange(1, 3001, dtype=np.int32) * 32
    assert host(mx.mx_check_offs(dev_i32(good), 3000 * 32, 32)).tolist() == [0, -1]


def sanitized(offs, m):
    out, prev = [], 0
    for e in offs:
        prev = min(max(int(e), prev), m)
        out.append(prev)
    return np.array(out, np.int32)


@pytest.mark.parametrize("bad", [
    [64, 32, 224 + 64],   # decreasing, last end beyond m
    [-64, 96, 224],       # negative first end
    [96, 96, 288],        # beyond m only
])
def test_gemm_out_of_contract_offs_stays_in_bounds(oracle, bad):
    rng = np.random.default_rng(5)
    m, n, k, G = 224, 64, 128, 3
    a_q, a_s = oracle.quantize_dim0(synth.normal_bf16(rng, (m, k), 1.0))
    b_q, b_s = oracle.quantize_dim0(synth.normal_bf16(rng, (G * n, k), 0.02))
    a_full = torch.zeros((m + 2 * GUARD, k), dtype=torch.uint8, device="cuda:0")
    a_full[GUARD:GUARD + m] = dev_u8(a_q)
    out_full = torch.full((m + 2 * GUARD, n), -7.0, dtype=torch.float32, device="cuda:0")
    offs = np.array(bad, np.int32)
    say(f"[offs out of contract] fwd offs={bad} m={m}")
    mx.mx_grouped_mm_fwd(a_full[GUARD:GUARD + m], dev_u8(oracle.scales_to_physical(a_s)), dev_u8(b_q),
                         dev_u8(oracle.scales_to_physical(b_s)), dev_i32(offs), m, n, k, out_dtype=mx.MX_OUT_F32,
                         out=out_full[GUARD:GUARD + m])
    got_full = host(out_full)
    assert np.all(got_full[:GUARD] == -7.0) and np.all(got_full[GUARD + m:] == -7.0), "a guard row was written"
    san = sanitized(offs, m)
    ref = oracle.mx_grouped_mm_fwd(a_q, a_s, b_q, b_s, san, G)
    rows = int(san[-1])
    got = got_full[GUARD:GUARD + rows]
    assert np.allclose(got, ref[:rows], rtol=1e-3, atol=1e-3), "rows of the sanitized groups"
    assert np.all(got_full[GUARD + rows:GUARD + m] == -7.0), "rows past the last (sanitized) group stay unwritten"
    # wgrad over token ranges past the contraction: clamped, nothing outside the operands
    a_t = torch.zeros((n + 2 * GUARD, m), dtype=torch.uint8, device="cuda:0")
    x_t = torch.zeros((k + 2 * GUARD, m), dtype=torch.uint8, device="cuda:0")
    s_t = torch.full((mx.mx_scale_bytes(n, m),), 127, dtype=torch.uint8, device="cuda:0")
    s_x = torch.full((mx.mx_scale_bytes(k, m),), 127, dtype=torch.uint8, device="cuda:0")
    dw = mx.mx_grouped_mm_wgrad(a_t[GUARD:GUARD + n], s_t, x_t[GUARD:GUARD + k], s_x, dev_i32(offs), m, n, k,
                                out_dtype=mx.MX_OUT_F32)
    assert not host(dw).any()  # zero operands: every group's (clamped) sum is zero
    torch.cuda.synchronize()
