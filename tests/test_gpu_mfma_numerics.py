"""The block-scaled MFMA's arithmetic, pinned bit for bit on constructed operands.

Each case below is one dot product whose exact value and whose value under the
run-of-eight truncation (tests/mfma_model.py) differ by a predicted amount; the
expected value is written out by hand for every case and also recomputed by the
model. The same cases run through
  * the library's grouped forward GEMM (m = n = 32, k = 64: one instruction per
    output; k = 128: two, accumulated in fp32), which uses the 32x32x64 form with
    the weight operand first, and
  * mx_probe_mfma_dot: one 32x32x64 and one 16x16x128 instruction, both operand
    orders.
Both full-rate forms and both operand orders give the same truncation, so no
full-rate arrangement of the instruction reaches an IEEE fp32 sum. A second test
bounds every output of realistic quantized data against the model.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import mxfp8_block_scaled_amd as mx

import mfma_model
from gpu_util import dev_u8, host, require_gpu, say
from mfma_cases import CASES, build

F = Fraction

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def _check_diag(d, R, label, record):
    n = min(R, len(CASES))
    wrong = []
    for i in range(n):
        name, _, want, why = CASES[i]
        got = F(float(d[i, i]))
        say(f"    [{label}] {name}: got {float(got)!r}, expected {float(want)!r} ({why})")
        if got != want:
            wrong.append(f"{name}: got {float(got)!r} expected {float(want)!r}")
    assert not wrong, f"{label}: " + "; ".join(wrong)
    record.append(label)


@pytest.fixture(scope="module")
def record():
    rec = []
    yield rec
    out = os.environ.get("MX_NUMERICS_RECORD")
    if out:
        with open(out, "a") as fh:
            fh.write(json.dumps({"test": "mfma_cases", "paths_bit_exact": rec, "cases": [c[0] for c in CASES]}) + "\n")


def test_cases_through_the_gemm(record):
    """The library's forward GEMM, k = 64: one 32x32x64 instruction per output."""
    import oracle.mx as orc

    a, sa, b, sb = build(32, 64)
    say("[mfma numerics] grouped fwd m=n=32 k=64")
    d = host(mx.mx_grouped_mm_fwd(dev_u8(a), dev_u8(orc.scales_to_physical(sa)), dev_u8(b),
                                  dev_u8(orc.scales_to_physical(sb)), None, 32, 32, 64, out_dtype=mx.MX_OUT_F32))
    _check_diag(d, 32, "gemm k=64", record)
    h, ab = mfma_model.run_truncated_mm(a, sa, b, sb)
    assert np.all(np.abs(d - h) <= mfma_model.tolerance(ab, 64) + 0.0)


def test_two_steps_through_the_gemm(record):
    """k = 128: case i in the first k-step and case i+1 in the second; the two
    instruction results add in the fp32 accumulator (exact here)."""
    import oracle.mx as orc

    a0, sa0, b0, sb0 = build(32, 64)
    n = len(CASES)
    perm = [(i + 1) % n for i in range(n)] + list(range(n, 32))
    a = np.concatenate([a0, a0[perm]], axis=1)
    b = np.concatenate([b0, b0[perm]], axis=1)
    sa = np.concatenate([sa0, sa0[perm]], axis=1)
    sb = np.concatenate([sb0, sb0[perm]], axis=1)
    say("[mfma numerics] grouped fwd m=n=32 k=128")
    d = host(mx.mx_grouped_mm_fwd(dev_u8(a), dev_u8(orc.scales_to_physical(sa)), dev_u8(b),
                                  dev_u8(orc.scales_to_physical(sb)), None, 32, 32, 128, out_dtype=mx.MX_OUT_F32))
    for i in range(n):
        want = CASES[i][2] + CASES[perm[i]][2]
        assert F(float(np.float32(float(want)))) == want
        assert F(float(d[i, i])) == want, f"two steps, cases {i} and {perm[i]}"
    record.append("gemm k=128")


@pytest.mark.parametrize("form", [mx.MX_PROBE_32X32X64, mx.MX_PROBE_32X32X64 | mx.MX_PROBE_SWAP,
                                  mx.MX_PROBE_16X16X128, mx.MX_PROBE_16X16X128 | mx.MX_PROBE_SWAP])
@pytest.mark.parametrize("shift", [0, 64])
def test_cases_one_instruction(form, shift, record):
    R, K = (16, 128) if form & 1 else (32, 64)
    if shift and not form & 1:
        pytest.skip("the 32x32x64 form contracts over 64 elements: nothing to shift into")
    a, sa, b, sb = build(R, K, shift=shift)
    say(f"[mfma numerics] probe form={form} shift={shift}")
    d = host(mx.mx_probe_mfma_dot(form, dev_u8(a), dev_u8(sa), dev_u8(b), dev_u8(sb)))
    _check_diag(d, R, f"form {form} shift {shift}", record)
    h, ab = mfma_model.run_truncated_mm(a, sa, b, sb)
    assert np.all(np.abs(d - h) <= mfma_model.LEVEL2 * ab)


def _quantized_rows(rng, R, K, sigma):
    import oracle.mx as orc
    from mxfp8_block_scaled_amd import synth

    return orc.quantize_dim0(synth.normal_bf16(rng, (R, K), sigma))


@pytest.mark.parametrize("form", [mx.MX_PROBE_32X32X64, mx.MX_PROBE_16X16X128])
def test_realistic_data_within_the_model(form):
    """N(0,1) x N(0,0.02) rows cast by the oracle: every instruction result lies within
    LEVEL2 * sum|ab| of the model; report how far the model and the hardware sit
    from the exact sum."""
    import oracle.mx as orc

    R, K = (16, 128) if form & 1 else (32, 64)
    rng = np.random.default_rng(7 + form)
    worst, fro_hw, fro_model, exact_hits, total = 0.0, [], [], 0, 0
    for trial in range(64):
        a, sa = _quantized_rows(rng, R, K, 1.0)
        b, sb = _quantized_rows(rng, R, K, 0.02)
        d = host(mx.mx_probe_mfma_dot(form, dev_u8(a), dev_u8(sa), dev_u8(b), dev_u8(sb))).astype(np.float64)
        h, ab = mfma_model.run_truncated_mm(a, sa, b, sb)
        ref = orc.dequantize(a, sa) @ orc.dequantize(b, sb).T
        worst = max(worst, float(np.max(np.abs(d - h) / ab)))
        exact_hits += int(np.sum(d == h.astype(np.float32)))
        total += d.size
        fro_hw.append(orc.rel_frobenius(d, ref))
        fro_model.append(orc.rel_frobenius(h, ref))
    say(f"    form {form}: max |hw - model| / sum|ab| = 2^{np.log2(worst) if worst else -99:.1f}; "
        f"{exact_hits}/{total} results equal the model rounded to fp32; rel. Frobenius vs exact: "
        f"hw {np.mean(fro_hw):.2e}, model {np.mean(fro_model):.2e}")
    out = os.environ.get("MX_NUMERICS_RECORD")
    if out:
        with open(out, "a") as fh:
            fh.write(json.dumps({"test": "mfma_realistic", "form": "16x16x128" if form & 1 else "32x32x64",
                                 "trials": 64, "results": total, "equal_model": exact_hits, "worst": worst,
                                 "fro_hw": float(np.mean(fro_hw)), "fro_model": float(np.mean(fro_model))}) + "\n")
    assert worst <= mfma_model.LEVEL2
