"""Pins for the oracle's cast (E4M3 table, RCEIL scale, encoder, the three forms).

Each check compares the oracle with something other than itself: a brute-force
search, a closed form derived from the bit layout, hand-worked values, or inputs
built so that the answer is known by construction.
"""

import math
import os

import numpy as np
import pytest

from mxfp8_block_scaled_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_values.txt")


def independent_e4m3_values():
    """E4M3 values built from integer significands (a different formula from the oracle's)."""
    vals = np.empty(256)
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        sig, ex = (m, -9) if e == 0 else (8 + m, e - 10)
        v = math.ldexp(sig, ex)
        if e == 15 and m == 7:
            v = math.nan
        vals[c] = -v if c & 0x80 else v
    return vals


def brute_force_encode(v):
    """argmin of |v - value| over the 127 non-negative finite codes, ties to the even code.

    Magnitudes >= 448 saturate to 0x7E; the sign bit of v (including -0.0) is copied.
    """
    v = np.asarray(v, dtype=np.float64)
    pv = independent_e4m3_values()[:0x7F]
    a = np.abs(v).ravel()
    uniq, inv = np.unique(a, return_inverse=True)
    d = np.abs(uniq[:, None] - pv[None, :])
    dmin = d.min(axis=1, keepdims=True)
    is_min = d == dmin
    n_min = is_min.sum(axis=1)
    first = np.argmax(is_min, axis=1)
    # two nearest codes: take the even one (a tie involves two adjacent codes)
    code = np.where((n_min > 1) & (first % 2 == 1), first + 1, first)
    code = np.where(uniq >= 448, 0x7E, code)
    out = code[inv].reshape(v.shape).astype(np.uint8)
    return out | (np.signbit(v).astype(np.uint8) << 7)


def test_e4m3_table_fixed_points(oracle):
    t = oracle.E4M3_TABLE
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0**-9  # smallest subnormal
    assert t[0x07] == 7 * 2.0**-9  # largest subnormal
    assert t[0x08] == 2.0**-6  # smallest normal
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(~np.isnan(t)) == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0..0x7E are increasing


def test_e4m3_table_matches_independent_formula(oracle):
    ind = independent_e4m3_values()
    t = oracle.E4M3_TABLE
    same = (t == ind) | (np.isnan(t) & np.isnan(ind))
    assert same.all()
    fin = ~np.isnan(t)
    assert np.array_equal(np.signbit(t[fin]), np.signbit(ind[fin]))


def test_encode_decode_roundtrip_every_code(oracle):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    v = oracle.e4m3_decode(codes)
    back = oracle.e4m3_encode(v, codes >> 7)
    assert np.array_equal(back, codes)


@pytest.mark.parametrize("s", [-127, -9, -3, 0, 1, 7, 120])
def test_encoder_matches_brute_force_all_bf16(oracle, s):
    """Every finite bf16 pattern, divided by 2^s, encodes like the brute-force argmin."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_to_f64(bits)
    fin = np.isfinite(x)
    v = np.ldexp(x[fin], -s)
    got = oracle.e4m3_encode(v, (bits[fin] >> 15).astype(np.int64))
    assert np.array_equal(got, brute_force_encode(v))


def closed_form_rceil_byte(bits):
    """RCEIL scale byte from the amax's bf16 bits (derived from the bit layout).

    amax = (1 + m/128) * 2^(E-127) for a normal value. 448 = 1.75 * 2^8, so
    amax/448 = ((1 + m/128) / 1.75) * 2^(E-135); the ratio lies in [1/1.75, 2/1.75),
    so ceil(log2) is E-135 for m <= 96 (ratio <= 1) and E-134 above. The byte is that
    plus 127, clamped at 0; denormal and zero amax clamp to 0.
    """
    E = (bits >> 7) & 0xFF
    m = bits & 0x7F
    byte = E.astype(np.int64) - 8 + (m > 0x60)
    byte = np.where(E == 0, 0, byte)
    return np.clip(byte, 0, 254)


def test_rceil_exhaustive_closed_form(oracle):
    bits = np.arange(0x7F80, dtype=np.uint32).astype(np.uint16)  # every non-negative finite bf16
    amax = oracle.bf16_to_f64(bits)
    got = oracle.rceil_exponent(amax) + 127
    assert np.array_equal(got, closed_form_rceil_byte(bits))


def test_rceil_log2_and_invariant(oracle):
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint32).astype(np.uint16)  # normal amax
    amax = oracle.bf16_to_f64(bits)
    s = oracle.rceil_exponent(amax)
    ref = np.array([max(-127, math.ceil(math.log2(a / 448.0))) for a in amax])
    assert np.array_equal(s, ref)
    un = s > -127
    ratio = amax[un] / np.ldexp(1.0, s[un])
    assert np.all((ratio > 224) & (ratio <= 448))
    # the largest finite bf16 stays far from the +127 clamp
    assert s.max() == 247 - 127


def test_rceil_vs_floor(oracle):
    """RCEIL = FLOOR + 1 exactly when amax's significand exceeds 1.75 (OCP FLOOR rule)."""
    bits = np.arange(0x0400, 0x7F80, dtype=np.uint32).astype(np.uint16)
    amax = oracle.bf16_to_f64(bits)
    s = oracle.rceil_exponent(amax)
    floor_s = np.floor(np.log2(amax)).astype(np.int64) - 8
    sig = amax / np.ldexp(1.0, np.floor(np.log2(amax)).astype(np.int64))
    assert np.array_equal(s, floor_s + (sig > 1.75))
    assert np.array_equal(oracle.floor_exponent(amax), floor_s)


def test_floor_exhaustive_closed_form(oracle):
    """FLOOR on every non-negative finite bf16 amax: from the bits, floor(log2 amax) is
    E - 127 for exponent field E >= 1, so s = E - 135, clamped at -127 (E = 0: zero or
    bf16-denormal amax, below 2^-126, clamps too); the block maximum over 2^s then
    lies in [256, 512) wherever s is not clamped."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    amax = oracle.bf16_to_f64(bits.astype(np.uint16))
    E = (bits >> 7).astype(np.int64)
    want = np.where(E == 0, -127, np.maximum(E - 135, -127))
    s = oracle.floor_exponent(amax)
    assert np.array_equal(s, want)
    pos = amax > 0
    assert np.array_equal(s[pos], np.clip(np.floor(np.log2(amax[pos])).astype(np.int64) - 8, -127, 127))
    free = s > -127
    ratio = amax[free] / np.ldexp(1.0, s[free])
    assert np.all((ratio >= 256) & (ratio < 512))
    # whole blocks: the scale byte of a block is s + 127 of its amax
    blk = np.zeros((bits.size, 32), np.uint16)
    blk[:, 5] = bits
    _, sb = oracle.quantize_blocks(blk, "floor")
    assert np.array_equal(sb.astype(np.int64), want + 127)


def test_floor_worked_values(oracle):
    """Worked by hand from floor(log2 amax) - 8 and the E4M3 grid (OCP MX FLOOR rule).

    amax 1.875 (bf16 0x3FF0): floor(log2) = 0, s = -8, byte 119; 1.875 * 2^8 = 480 > 448
    saturates to 0x7E (RCEIL gives byte 120 and 0x77 for the same block).
    amax 1.0: s = -8, byte 119, 1.0 -> 256 = 2^8 -> code 0x78.
    [2.5, 1.0]: floor(log2 2.5) = 1, s = -7, byte 120; 2.5 -> 320 = 1.25 * 2^8 -> 0x7A;
    1.0 -> 128 -> 0x70.
    [-448.0] (0xC3E0): floor(log2 448) = 8, s = 0, byte 127, code 0x80 | 0x7E = 0xFE.
    zero block: byte 0, codes 0 (the sign of zero kept).
    bf16 0x0040 = (64/128) * 2^-126 = 2^-127, a bf16 denormal: s clamps to -127 (byte 0)
    and the element encodes 2^-127 / 2^-127 = 1.0 -> 0x38.
    """
    def one(vals):
        blk = np.zeros((1, 32), np.uint16)
        blk[0, : len(vals)] = vals
        c, sb = oracle.quantize_blocks(blk, "floor")
        return [int(x) for x in c[0, : len(vals)]], int(sb[0])

    assert one([0x3FF0]) == ([0x7E], 119)
    assert one([0x3F80]) == ([0x78], 119)
    assert one([0x4020, 0x3F80]) == ([0x7A, 0x70], 120)
    assert one([0xC3E0]) == ([0xFE], 127)
    assert one([0x0000, 0x8000]) == ([0x00, 0x80], 0)
    assert one([0x0040]) == ([0x38], 0)
    # the same blocks under RCEIL, for contrast: 1.875 -> byte 120 and 1.875 * 2^7 = 240 -> 0x77
    c, sb = oracle.quantize_blocks(np.array([[0x3FF0] + [0] * 31], np.uint16), "rceil")
    assert (int(c[0, 0]), int(sb[0])) == (0x77, 120)


def parse_block(spec):
    parts = dict(p.split("=") for p in spec.split(","))
    if "fill" in parts:
        return np.full(32, int(parts["fill"], 16), dtype=np.uint16)
    blk = np.full(32, int(parts["rest"], 16), dtype=np.uint16)
    blk[0] = int(parts["one"], 16)
    return blk


def test_worked_values(oracle):
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        blk_s, byte_s, elem_s = [p.strip() for p in line.split("|")]
        x_hex, code_hex = [p.strip() for p in elem_s.split("->")]
        blk = parse_block(blk_s)
        codes, scales = oracle.quantize_blocks(blk[None, :])
        assert int(scales[0]) == int(byte_s), line
        idx = int(np.flatnonzero(blk == int(x_hex, 16))[0])
        assert int(codes[0, idx]) == int(code_hex, 16), line
        n += 1
    assert n >= 12


def test_outlier_dequantizes_to_10240(oracle):
    codes, scales = oracle.quantize_blocks(np.full((1, 32), 0x461C, np.uint16))
    assert oracle.dequantize(codes, scales[:, None])[0, 0] == 10240.0


def roundtrip_blocks(rng, nblocks, s_lo=-100, s_hi=100):
    """Blocks built as code values x 2^s with the largest magnitude in (224, 448]."""
    vals = independent_e4m3_values()
    codes = rng.integers(0, 0x7F, size=(nblocks, 32)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=(nblocks, 32)) << 7).astype(np.uint8)
    codes[codes == 0x7F] = 0x10
    codes[codes == 0xFF] = 0x90
    big = rng.integers(0x77, 0x7F, size=nblocks).astype(np.uint8)  # 240..448 (0x76 is 224)
    pos = rng.integers(0, 32, size=nblocks)
    codes[np.arange(nblocks), pos] = big | (codes[np.arange(nblocks), pos] & 0x80)
    s = rng.integers(s_lo, s_hi, size=nblocks)
    x = np.ldexp(vals[codes], s[:, None]).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    assert np.array_equal(synth.bf16_bits_to_f32(bits), x)  # representable exactly
    return bits, codes, (s + 127).astype(np.uint8)


def test_roundtrip_representable_blocks(oracle):
    rng = np.random.default_rng(11)
    bits, codes, sbytes = roundtrip_blocks(rng, 4000)
    q, s = oracle.quantize_blocks(bits)
    assert np.array_equal(s, sbytes)
    assert np.array_equal(q, codes)


def test_special_blocks(oracle):
    z = np.zeros((2, 32), np.uint16)
    z[1, 5] = 0x8000
    q, s = oracle.quantize_blocks(z)
    assert np.all(s == 0) and q[1, 5] == 0x80 and np.sum(q != 0) == 1
    den = np.array([[0x0001] * 16 + [0x8003] * 16], np.uint16)  # 2^-133 and -3*2^-133
    q, s = oracle.quantize_blocks(den)
    assert s[0] == 0
    assert np.all(q[0, :16] == 0x08)  # 2^-6
    assert np.all(q[0, 16:] == 0x94)  # -3*2^-6 = -1.5*2^-5 -> exponent field 2, mantissa 4


def test_dim0_matches_per_block(oracle):
    rng = np.random.default_rng(3)
    bits, codes, sbytes = roundtrip_blocks(rng, 6 * 8)
    x = bits.reshape(6, 8 * 32)
    q, s = oracle.quantize_dim0(x)
    assert np.array_equal(q, codes.reshape(6, 256))
    assert np.array_equal(s, sbytes.reshape(6, 8))


def test_dim1_blocks_run_down_columns(oracle):
    """Blocks built along the columns of X come back as rows of the transposed output."""
    rng = np.random.default_rng(4)
    R, C = 96, 40
    bits, codes, sbytes = roundtrip_blocks(rng, C * (R // 32))
    # block (c, j) holds X[32j:32j+32, c]
    x = np.empty((R, C), np.uint16)
    blk = bits.reshape(C, R // 32, 32)
    for c in range(C):
        for j in range(R // 32):
            x[32 * j:32 * j + 32, c] = blk[c, j]
    q_t, s_t = oracle.quantize_dim1(x)
    assert q_t.shape == (C, R) and s_t.shape == (C, R // 32)
    assert np.array_equal(q_t, codes.reshape(C, R))
    assert np.array_equal(s_t, sbytes.reshape(C, R // 32))


def test_weight_32x32(oracle):
    rng = np.random.default_rng(5)
    N, K = 64, 96
    w = synth.normal_bf16(rng, (N, K), 0.02)
    w[0:32, 32:64] = 0  # one all-zero tile
    q, q_t, s_row, s_col = oracle.quantize_weight_32x32(w)
    assert np.array_equal(q_t, q.T)
    _, s0 = oracle.quantize_dim0(w)
    for tn in range(N // 32):
        for tk in range(K // 32):
            tile_byte = s_row[32 * tn, tk]
            # the tile scale is the largest of its 32 row-block scales (RCEIL is monotone)
            assert tile_byte == s0[32 * tn:32 * tn + 32, tk].max()
            assert np.all(s_row[32 * tn:32 * tn + 32, tk] == tile_byte)
            assert np.all(s_col[32 * tk:32 * tk + 32, tn] == tile_byte)
            # every element of the tile is encoded with the tile scale
            x = oracle.bf16_to_f64(w[32 * tn:32 * tn + 32, 32 * tk:32 * tk + 32])
            v = np.ldexp(x, -(int(tile_byte) - 127))
            ref = brute_force_encode(v.ravel()).reshape(32, 32)
            assert np.array_equal(q[32 * tn:32 * tn + 32, 32 * tk:32 * tk + 32], ref)
    assert s_row[0, 1] == 0  # the zero tile


def test_nonfinite_reading(oracle):
    """NaN / Inf handling (a reading; parity unpinned, the HIP path requires finite input)."""
    b = np.full((2, 32), 0x3F80, np.uint16)
    b[0, 3] = 0x7FC0  # NaN
    b[1, 4] = 0xFF80  # -Inf
    q, s = oracle.quantize_blocks(b)
    assert s[0] == 0xFF and np.all(q[0] == 0x7F)
    assert s[1] == 254 and q[1, 4] == 0xFE
