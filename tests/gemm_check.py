"""Numerical bars for the GEMM parity tests, all against the float64 product of the
same dequantized operands (shared by the small and the full-size tests):
  * every fp32 output within HW_REL * sum_k |a_k b_k| (+ the fp32 accumulation
    bound). The gfx950 block-scaled MFMA does not round each addition to fp32:
    inside one 64-element dot product it drops product bits below about 2^-14 of
    the largest product (measured on adversarial random codes: worst error
    3.2e-4 = 2^-11.6 of sum |a b| per instruction). HW_REL = 2^-11 covers that;
  * relative Frobenius error reported for every case and held to REL_FRO_HW plus
    the growth of fp32 accumulation rounding with the contraction (rel_fro_gate);
  * bf16 output within 1 bf16 ulp of the correctly rounded value, or inside the
    per-element bound above plus half a bf16 ulp.
"""

import numpy as np

from gpu_util import say

REL_FRO = 1e-5  # the bound an IEEE fp32 accumulation would meet (reported, not gated)
REL_FRO_HW = 5e-5  # gate: measured 1.5e-5 on N(0,1) x N(0,0.02) data, K = 512
HW_REL = 2.0**-11


def rel_fro_gate(K):
    """The Frobenius gate for a contraction of length K: REL_FRO_HW (measured at
    K = 512) plus the growth of the accumulator's own rounding, one fp32 rounding
    per 64-element MFMA k-step; n such roundings walk randomly to about sqrt(n) u,
    and 8 u per sqrt(step) leaves room for the instruction's internal truncation.
    At K = 4096 the gate is 5.4e-5, at K = 2^22 1.7e-4."""
    if not K:
        return REL_FRO_HW
    return REL_FRO_HW + (K / 64) ** 0.5 * 2.0**-21


def check_f32(oracle, got, ref, name, absprod=None, K=None):
    err = oracle.rel_frobenius(got, ref)
    gate = rel_fro_gate(K)
    say(f"    {name}: rel frobenius {err:.3e} (gate {gate:.2e}; IEEE-fp32 bar {REL_FRO:g}: "
        f"{'met' if err <= REL_FRO else 'not met'})")
    assert err <= gate, f"{name}: relative Frobenius error {err:.3e} > {gate:.2e}"
    if absprod is not None:
        u = 2.0**-24
        bound = (HW_REL + K * u / (1 - K * u)) * absprod + 1e-30
        worst = np.max(np.abs(got - ref) / bound)
        say(f"    {name}: worst |err| / per-element bound = {worst:.3f}")
        assert worst <= 1.0, f"{name}: per-element bound exceeded ({worst:.3f})"


def check_bf16(oracle, got_bits, ref, absprod, K, name):
    """R13 rule: ordinal distance <= 1 from RNE_bf16(ref), else |err| within gamma_K * sum|a||b|."""
    ref_bits = oracle.round_to_bf16_bits(ref)
    d = np.abs(oracle.bf16_ordinal(got_bits) - oracle.bf16_ordinal(ref_bits))
    bad = d > 1
    if bad.any():
        got = oracle.bf16_to_f64(got_bits[bad])
        u = 2.0**-24
        gamma = K * u / (1 - K * u)
        # the bf16 rounding of the fp32 result adds half a bf16 ulp
        bound = (HW_REL + gamma) * absprod[bad] + np.abs(ref[bad]) * 2.0**-8
        assert np.all(np.abs(got - ref[bad]) <= bound), f"{name}: {np.sum(np.abs(got - ref[bad]) > bound)} outside bound"
    say(f"    {name}: {bad.sum()} of {d.size} outputs needed the fp32-bound branch")
