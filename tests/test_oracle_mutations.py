"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutant below replaces one oracle function with a subtly wrong version; the
named pin must then fail. This shows the pins constrain each step of the oracle,
not just its overall shape.
"""

import numpy as np
import pytest

from oracle import mx

import test_oracle_cast as tc
import test_oracle_gemm as tg
import test_oracle_layout as tl
import test_oracle_pad as tp
import test_oracle_backward as tb


def enc_ties_away(v, negative):
    a = np.abs(np.asarray(v, dtype=np.float64))
    pv = mx.E4M3_TABLE[:0x7F]
    lo = np.clip(np.searchsorted(pv, a, side="right") - 1, 0, 0x7E)
    hi = np.clip(lo + 1, 0, 0x7E)
    code = np.where(a - pv[lo] < pv[hi] - a, lo, hi)  # ties go up
    code = np.where(a >= 448, 0x7E, code)
    return (code | (np.asarray(negative, dtype=np.int64) << 7)).astype(np.uint8)


def enc_no_saturation(v, negative):
    a = np.abs(np.asarray(v, dtype=np.float64))
    out = mx.__dict__["_orig_encode"](v, negative)
    return np.where(a > 448, 0x7F | (np.asarray(negative, dtype=np.int64) << 7), out).astype(np.uint8)


def enc_drop_sign_of_zero(v, negative):
    out = mx.__dict__["_orig_encode"](v, negative)
    return np.where((out & 0x7F) == 0, 0, out).astype(np.uint8)


def rceil_floor(amax):
    amax = np.asarray(amax, dtype=np.float64)
    a = np.where(amax > 0, amax, 1.0)
    s = np.floor(np.log2(a)).astype(np.int64) - 8
    return np.clip(np.where(amax == 0, -127, s), -127, 127)


def floor_via_ceil(amax):
    amax = np.asarray(amax, dtype=np.float64)
    a = np.where(amax > 0, amax, 1.0)
    s = np.ceil(np.log2(a)).astype(np.int64) - 8
    return np.clip(np.where(amax == 0, -127, s), -127, 127)


def floor_emax_7(amax):
    return np.clip(mx.__dict__["_orig_floor"](amax) + 1, -127, 127)


def rceil_off_by_one(amax):
    return np.clip(mx.__dict__["_orig_rceil"](amax) + 1, -127, 127)


def offset_swapped(r, kb, KB):
    kt = -(-KB // 8)
    return ((r // 32) * kt + kb // 8) * 256 + ((kb % 8) // 2) * 64 + (r % 32) * 2 + (kb % 2)


def group_bounds_shifted(offs, total):
    if offs is None:
        return [(0, total)]
    offs = [int(o) for o in offs]
    starts = [0] + [o + 1 for o in offs[:-1]]
    return list(zip(starts, offs))


def wgrad_misaligned_rows(a_t, b_t, offs, groups):
    """Pairs row r of dY^T with row r+1 of X^T inside each group (a wrong index)."""
    N, M = a_t.shape
    K = b_t.shape[0]
    out = np.zeros((groups, N, K))
    for g, (r0, r1) in enumerate(mx.group_bounds(offs, M)):
        if r1 > r0:
            idx = np.minimum(np.arange(r0, r1) + 1, M - 1)
            out[g] = a_t[:, r0:r1] @ b_t[:, idx].T
    return out


def dequant_bias128(q, scales):
    s = np.asarray(scales, dtype=np.int64) - 128
    return mx.e4m3_decode(q) * np.repeat(np.ldexp(1.0, s), 32, axis=1)


def bf16_round_via_f32(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def padded_offsets_round_down(offs):
    out, total = [], 0
    for start, end in mx.group_bounds(offs, None):
        total += ((end - start) // 32) * 32
        out.append(total)
    return out


def padded_rows_no_growth(rows, groups):
    return ((rows + 31) // 32) * 32


def pad_at_unpadded_start(x, offs, rows_pad):
    """Moves each group to its unpadded start instead of its padded one."""
    x = np.asarray(x)
    out = np.zeros((rows_pad,) + x.shape[1:], dtype=x.dtype)
    for start, end in mx.group_bounds(offs, None):
        out[start:end] = x[start:end]
    return out, mx.padded_offsets(offs)


def unpad_from_previous_group(y_pad, offs, rows):
    """Reads group g from the padded run of group g - 1's end (an off-by-one group)."""
    y_pad = np.asarray(y_pad)
    ends = mx.padded_offsets(offs)
    out = np.zeros((rows,) + y_pad.shape[1:], dtype=y_pad.dtype)
    for g, (start, end) in enumerate(mx.group_bounds(offs, None)):
        base = ends[g - 2] if g >= 2 else 0
        out[start:end] = y_pad[base:base + end - start]
    return out


def transpose_whole_stack(w, groups):
    """Transposes the stacked [G * N, K] weight as one matrix and cuts it into
    groups along the wrong axis."""
    w = np.asarray(w, dtype=np.float64)
    N = w.shape[0] // groups
    t = w.T  # [K, G * N]
    return np.concatenate([t[:, g * N:(g + 1) * N].T.reshape(-1, N)[: t.shape[0]] for g in range(groups)])


def dequant_bf16_truncating(q, scales):
    f = mx.dequantize(q, scales).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


MUTANTS = [
    ("e4m3_encode", enc_ties_away, tc.test_encoder_matches_brute_force_all_bf16, {"s": 0}),
    ("e4m3_encode", enc_ties_away, tc.test_worked_values, {}),
    ("e4m3_encode", enc_no_saturation, tc.test_encoder_matches_brute_force_all_bf16, {"s": -127}),
    ("e4m3_encode", enc_drop_sign_of_zero, tc.test_special_blocks, {}),
    ("rceil_exponent", rceil_floor, tc.test_rceil_exhaustive_closed_form, {}),
    ("rceil_exponent", rceil_floor, tc.test_worked_values, {}),
    ("rceil_exponent", rceil_off_by_one, tc.test_roundtrip_representable_blocks, {}),
    ("floor_exponent", floor_via_ceil, tc.test_floor_exhaustive_closed_form, {}),
    ("floor_exponent", floor_emax_7, tc.test_floor_worked_values, {}),
    ("scale_offset", offset_swapped, tl.test_layout_feeds_mfma_lanes, {}),
    ("group_bounds", group_bounds_shifted, tg.test_grouped_mm_matches_loops, {}),
    ("grouped_mm_wgrad", wgrad_misaligned_rows, tg.test_wgrad_matches_loops_and_empty_group_is_zero, {}),
    ("dequantize", dequant_bias128, tg.test_exact_integer_case_matches_rationals, {}),
    ("round_to_bf16_bits", bf16_round_via_f32, tg.test_bf16_rounding, {}),
    ("padded_offsets", padded_offsets_round_down, tp.test_golden_cases, {}),
    ("padded_rows", padded_rows_no_growth, tp.test_size_bound_exhaustive, {}),
    ("pad_token_groups", pad_at_unpadded_start, tp.test_padded_wgrad_equals_per_group_brute_force, {}),
    ("unpad_token_groups", unpad_from_previous_group, tp.test_pad_properties, {"seed": 1}),
    ("_per_group_transpose", transpose_whole_stack, tb.test_backward_matches_loops, {}),
    ("dequantize_to_bf16_bits", dequant_bf16_truncating, tb.test_dequantize_to_bf16_every_code_and_scale, {}),
]


@pytest.mark.parametrize("name,mutant,pin,kwargs", MUTANTS, ids=[f"{m[0]}-{m[1].__name__}" for m in MUTANTS])
def test_pin_catches_mutant(monkeypatch, name, mutant, pin, kwargs):
    monkeypatch.setitem(mx.__dict__, "_orig_encode", mx.e4m3_encode)
    monkeypatch.setitem(mx.__dict__, "_orig_rceil", mx.rceil_exponent)
    monkeypatch.setitem(mx.__dict__, "_orig_floor", mx.floor_exponent)
    monkeypatch.setattr(mx, name, mutant)
    with pytest.raises(AssertionError):
        pin(mx, **kwargs)


def test_unmutated_pins_pass():
    tc.test_encoder_matches_brute_force_all_bf16(mx, 0)
    tl.test_layout_feeds_mfma_lanes(mx)
    tg.test_exact_integer_case_matches_rationals(mx)
