"""Plain CPU oracle for the MXFP8 training cast and the MXFP8 scaled grouped GEMM.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this module: only the test suite, the smoke check and the CPU-baseline leg of the
benchmark use it. It shares no code, table or constant with the HIP library.

Everything is numpy in float64, which holds every bf16 input, every E4M3 value,
every E8M0 scale and every product of the two exactly, so each step below is exact
except the final summation order of a matmul.

What is computed (sources):
  * The cast: bf16 in, 32-element blocks, block amax, an E8M0 scale rounded up
    ("RCEIL"), E4M3 codes, saturating. The pages name the pieces -- 1x32 blocks,
    RCEIL, blocked E8M0 scales, dim0/dim1 casts and the 32x32 weight-scale policy
    (torchtitan PR 5334 body; ao fork PR 10 "Design notes" and "Numerics
    evidence") -- but print no formula. The formula is the OCP Microscaling (MX)
    definition: the scale exponent is ceil(log2(amax / 448)), 448 being the largest
    E4M3 value, and elements are encoded round-to-nearest-even with saturation.
    The OCP default scale rule, FLOOR, is kept beside it (ao fork PR 10, "Known
    follow-ups": FLOOR is reachable but untested there): the exponent is
    floor(log2(amax)) - 8, 8 being the exponent of E4M3's largest power of two,
    so the block maximum can land in [256, 512) and saturate to 448.
  * The GEMM: a grouped matmul over per-group row offsets `offs` (ao fork PR 10
    "Summary"; pytorch/ao PR 4705 body), with offs=None meaning one dense group
    (torchtitan PR 5334 body), in forward, dgrad and wgrad form.
  * The backward override arms: gradients from the saved bf16 operands, or from
    the dequantized forward operands, through bf16 grouped GEMMs (ao fork PR 10,
    "Design notes" and review pass).
  * Token-group padding: each group's token rows moved to a run that starts at a
    multiple of 32, the rest zero, and the inverse gather (pytorch/ao PR 4705,
    ghstack list: pad/unpad kernels; ao fork PR 10, "Known follow-ups").

Readings where the pages are silent (each also listed in the design notes):
  * a zero block gets scale byte 0 (the clamp of -inf to the E8M0 floor -127);
  * blocks whose amax is tiny clamp to scale byte 0 and keep their (non-zero)
    codes, i.e. x * 2^127 is encoded, nothing is flushed;
  * the sign of zero is kept (-0.0 -> 0x80);
  * NaN anywhere in a block -> scale 0xFF and every code 0x7F; +-Inf with no NaN
    -> scale byte 254 and +-448 for the infinite elements. (parity unpinned: the
    HIP library requires finite input and is not compared on this.)
  * the 32x32 weight form keeps ONE code array, quantized with each 32x32 tile's
    scale; its transpose is the column-major copy.
"""

import numpy as np

# --------------------------------------------------------------------------------------
# bf16 and E4M3 decoding (OCP MX: E4M3 has 1 sign, 4 exponent bits with bias 7, 3
# mantissa bits, no infinities, NaN = S.1111.111, largest finite value 448).
# --------------------------------------------------------------------------------------

E4M3_MAX = 448.0
SCALE_BIAS = 127
SCALE_MIN_EXP = -127  # E8M0 byte 0
SCALE_MAX_EXP = 127  # E8M0 byte 254 (255 is NaN)
BLOCK = 32


def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns (uint16 array) as float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_value(code):
    """Value of one E4M3 code (int 0..255), from the format's field definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = m * 2.0**-9  # subnormal: m/8 * 2^(1-7)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return sign * mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# finite non-negative codes 0x00..0x7E, in increasing order of value
_POS_CODES = np.arange(0x7F)
_POS_VALUES = E4M3_TABLE[:0x7F]


def e4m3_decode(codes):
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# --------------------------------------------------------------------------------------
# Scale (RCEIL) and element encoding
# --------------------------------------------------------------------------------------


def rceil_exponent(amax):
    """Smallest integer s with amax <= 448 * 2^s, clamped to [-127, 127].

    This is ceil(log2(amax / 448)) (OCP MX scale rule with rounding up), evaluated
    without a logarithm: start below the answer, from the binary exponent of amax,
    and step up until the defining inequality holds, then check it fails one step
    lower. amax = 0 gives the clamp of -inf, i.e. -127; +Inf clamps to 127.
    Accepts a scalar or an array of non-negative float64 values; returns int64.
    """
    amax = np.asarray(amax, dtype=np.float64)
    finite_pos = np.isfinite(amax) & (amax > 0)
    a = np.where(finite_pos, amax, 1.0)
    _, e = np.frexp(a)  # a = f * 2^e with f in [0.5, 1)
    s = e.astype(np.int64) - 10
    while True:
        up = a > E4M3_MAX * np.ldexp(1.0, s)
        if not up.any():
            break
        s = np.where(up, s + 1, s)
    assert not (a <= E4M3_MAX * np.ldexp(1.0, s - 1)).any()
    s = np.where(amax == 0, SCALE_MIN_EXP, s)
    s = np.where(np.isinf(amax), SCALE_MAX_EXP, s)
    return np.clip(s, SCALE_MIN_EXP, SCALE_MAX_EXP)


def floor_exponent(amax):
    """floor(log2(amax)) - 8, clamped to [-127, 127] (the OCP MX FLOOR scale rule).

    floor(log2(a)) is read off the binary exponent: a = f * 2^e with f in [0.5, 1)
    gives floor(log2(a)) = e - 1 exactly. amax = 0 gives the clamp of -inf, i.e.
    -127; +Inf clamps to 127. Accepts a scalar or an array of non-negative float64
    values; returns int64.
    """
    amax = np.asarray(amax, dtype=np.float64)
    finite_pos = np.isfinite(amax) & (amax > 0)
    a = np.where(finite_pos, amax, 1.0)
    _, e = np.frexp(a)
    s = e.astype(np.int64) - 1 - 8
    s = np.where(amax == 0, SCALE_MIN_EXP, s)
    s = np.where(np.isinf(amax), SCALE_MAX_EXP, s)
    return np.clip(s, SCALE_MIN_EXP, SCALE_MAX_EXP)


def scale_exponent(amax, scale_mode):
    """The block scale exponent under `scale_mode` ("rceil" or "floor")."""
    if scale_mode == "rceil":
        return rceil_exponent(amax)
    if scale_mode == "floor":
        return floor_exponent(amax)
    raise ValueError(f"unknown scale mode {scale_mode!r}")


def e4m3_encode(v, negative):
    """Round-to-nearest-even, saturating E4M3 encode of float64 values `v`.

    `negative` carries the sign bit separately so that -0.0 (and negative values
    that round to zero) keep it. |v| >= 448 saturates to the largest finite code.
    Ties go to the code whose mantissa LSB is 0; for E4M3 that is the even code.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    lo = np.searchsorted(_POS_VALUES, a, side="right") - 1  # largest code with value <= a
    lo = np.clip(lo, 0, 0x7E)
    hi = np.clip(lo + 1, 0, 0x7E)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | (np.asarray(negative, dtype=np.int64) << 7)
    return code.astype(np.uint8)


def quantize_blocks(bits, scale_mode="rceil"):
    """Quantize a [nblocks, blocksize] array of bf16 patterns, one scale per row.

    scale_mode: "rceil" (the pages' rule) or "floor" (the OCP default).
    Returns (codes uint8 [nblocks, blocksize], scale bytes uint8 [nblocks]).
    """
    bits = np.asarray(bits, dtype=np.uint16)
    x = bf16_to_f64(bits)
    neg = (bits >> 15).astype(np.int64)
    nb = x.shape[0]
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(nb, dtype=np.uint8)
    has_nan = np.isnan(x).any(axis=1)
    amax = np.where(np.isnan(x), 0.0, np.abs(x)).max(axis=1) if x.shape[1] else np.zeros(nb)
    exps = scale_exponent(amax, scale_mode)
    scales[:] = (exps + SCALE_BIAS).astype(np.uint8)
    v = np.ldexp(x, -exps[:, None])  # exact: a power-of-two scale
    codes[:] = e4m3_encode(v, neg)
    codes[has_nan] = 0x7F
    scales[has_nan] = 0xFF
    return codes, scales


# --------------------------------------------------------------------------------------
# The three cast forms
# --------------------------------------------------------------------------------------


def quantize_dim0(bits, scale_mode="rceil"):
    """1x32 rowwise cast of a [R, C] bf16 matrix (C % 32 == 0): blocks run along C.

    Returns q uint8 [R, C] and logical scales uint8 [R, C/32].
    """
    bits = np.asarray(bits, dtype=np.uint16)
    R, C = bits.shape
    assert C % BLOCK == 0
    codes, scales = quantize_blocks(bits.reshape(R * C // BLOCK, BLOCK), scale_mode)
    return codes.reshape(R, C), scales.reshape(R, C // BLOCK)


def quantize_dim1(bits, scale_mode="rceil"):
    """32x1 columnwise cast of a [R, C] bf16 matrix (R % 32 == 0): blocks run along R.

    The output is transposed so that the blocked axis is contiguous: q_t [C, R] and
    logical scales [C, R/32]. By definition this is dim0 of the transpose.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return quantize_dim0(np.ascontiguousarray(bits.T), scale_mode)


def quantize_weight_32x32(bits):
    """32x32 weight cast of W [N, K] (N % 32 == 0, K % 32 == 0).

    One scale per 32x32 tile, computed from the tile's amax; every element of the
    tile is encoded with it. Returns
      q      uint8 [N, K]       rowwise codes (feeds Y = X W^T)
      q_t    uint8 [K, N]       the same codes transposed (feeds dX = dY W)
      s_row  uint8 [N, K/32]    logical scales of q   (tile byte repeated over 32 rows)
      s_col  uint8 [K, N/32]    logical scales of q_t (tile byte repeated over 32 cols)
    """
    bits = np.asarray(bits, dtype=np.uint16)
    N, K = bits.shape
    assert N % BLOCK == 0 and K % BLOCK == 0
    tiles = bits.reshape(N // BLOCK, BLOCK, K // BLOCK, BLOCK).transpose(0, 2, 1, 3)
    codes, scales = quantize_blocks(tiles.reshape(-1, BLOCK * BLOCK))
    codes = codes.reshape(N // BLOCK, K // BLOCK, BLOCK, BLOCK).transpose(0, 2, 1, 3).reshape(N, K)
    tile_s = scales.reshape(N // BLOCK, K // BLOCK)
    s_row = np.repeat(tile_s, BLOCK, axis=0)  # [N, K/32]
    s_col = np.repeat(tile_s.T, BLOCK, axis=0)  # [K, N/32]
    return codes, np.ascontiguousarray(codes.T), s_row, s_col


def dequantize(q, scales):
    """value(code) * 2^(byte - 127), float64, for q [R, C] and logical scales [R, C/32]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.int64) - SCALE_BIAS
    vals = e4m3_decode(q)
    return vals * np.repeat(np.ldexp(1.0, s), BLOCK, axis=1)


# --------------------------------------------------------------------------------------
# Physical scale layout: the GEMM-ready ("blocked") arrangement the cast writes.
#
# A logical scale array [R, KB] (KB = C/32 blocks per row) is stored as tiles of
# 32 rows x 8 blocks, 256 bytes each, tiles ordered row-tile major:
#   tile   = (r // 32) * ceil(KB / 8) + kb // 8
#   offset = tile * 256 + (kb % 2) * 128 + (r % 32) * 4 + (kb % 8) // 2
# Bytes that no (r, kb) maps to (rows past R, blocks past KB) hold 0x7F.
# This is an independent restatement of the layout the library documents.
# --------------------------------------------------------------------------------------

SCALE_PAD = 0x7F


def scale_tiles(R, KB):
    return -(-R // 32), -(-KB // 8)


def scale_bytes(R, KB):
    rt, kt = scale_tiles(R, KB)
    return rt * kt * 256


def scale_offset(r, kb, KB):
    _, kt = scale_tiles(1, KB)
    return ((r // 32) * kt + kb // 8) * 256 + (kb % 2) * 128 + (r % 32) * 4 + (kb % 8) // 2


def scales_to_physical(logical):
    logical = np.asarray(logical, dtype=np.uint8)
    R, KB = logical.shape
    out = np.full(scale_bytes(R, KB), SCALE_PAD, dtype=np.uint8)
    r, kb = np.meshgrid(np.arange(R), np.arange(KB), indexing="ij")
    out[scale_offset(r, kb, KB)] = logical
    return out


def scales_from_physical(phys, R, KB):
    phys = np.asarray(phys, dtype=np.uint8)
    r, kb = np.meshgrid(np.arange(R), np.arange(KB), indexing="ij")
    return phys[scale_offset(r, kb, KB)]


# --------------------------------------------------------------------------------------
# Grouped GEMM (float64)
# --------------------------------------------------------------------------------------


def group_bounds(offs, total):
    """Half-open row ranges of each group: group g = [offs[g-1], offs[g]), offs[-1] = 0.

    offs=None means one dense group covering all `total` rows.
    """
    if offs is None:
        return [(0, total)]
    offs = [int(o) for o in offs]
    starts = [0] + offs[:-1]
    return list(zip(starts, offs))


def grouped_mm(a, b, offs, groups):
    """C[r, :] = a[r, :] @ b_g^T for every row r of group g (float64 operands).

    a: [M, K]; b: [G * N, K] (the G per-group [N, K] matrices stacked); returns
    [M, N]. This is forward (a = X, b = W) and, with a = dY and b = W^T per group,
    dgrad. Rows outside every group stay zero.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    M, K = a.shape
    N = b.shape[0] // groups
    out = np.zeros((M, N), dtype=np.float64)
    for g, (r0, r1) in enumerate(group_bounds(offs, M)):
        if r1 > r0:
            out[r0:r1] = a[r0:r1] @ b[g * N:(g + 1) * N].T
    return out


def grouped_mm_wgrad(a_t, b_t, offs, groups):
    """dW_g = a_t[:, rows_g] @ b_t[:, rows_g]^T for each group (float64).

    a_t: [N, M] (dY^T), b_t: [K, M] (X^T); the contraction runs over the group's
    rows. Returns [G, N, K]; an empty group gives zeros.
    """
    a_t = np.asarray(a_t, dtype=np.float64)
    b_t = np.asarray(b_t, dtype=np.float64)
    N, M = a_t.shape
    K = b_t.shape[0]
    out = np.zeros((groups, N, K), dtype=np.float64)
    for g, (r0, r1) in enumerate(group_bounds(offs, M)):
        if r1 > r0:
            out[g] = a_t[:, r0:r1] @ b_t[:, r0:r1].T
    return out


def mx_grouped_mm_fwd(a_q, a_s, b_q, b_s, offs, groups):
    """Forward on quantized operands: dequantize both, then grouped_mm."""
    return grouped_mm(dequantize(a_q, a_s), dequantize(b_q, b_s), offs, groups)


def mx_grouped_mm_wgrad(a_tq, a_ts, b_tq, b_ts, offs, groups):
    return grouped_mm_wgrad(dequantize(a_tq, a_ts), dequantize(b_tq, b_ts), offs, groups)


# --------------------------------------------------------------------------------------
# Backward override arms (bf16 grouped GEMMs)
# --------------------------------------------------------------------------------------
#
# ao fork PR 10 ("Design notes") lets the backward of the MXFP8 grouped GEMM come
# from elsewhere while the quantized forward stays as it is: "high_precision" takes
# both gradients from the saved bf16 operands with plain bf16 grouped GEMMs;
# "dequantized" dequantizes the saved quantized forward operands (the dim0 codes and
# their logical scales) and runs the same two GEMMs, so the gradients belong to the
# function the quantized forward computes; the review pass of that page also names a
# wgrad-only high-precision switch. A bf16 grouped GEMM multiplies bf16 operands and
# accumulates in fp32; its exact value is the float64 product below.


def dequantize_to_bf16_bits(q, scales):
    """value(code) * 2^(byte - 127) rounded to bf16 (round-to-nearest-even)."""
    return round_to_bf16_bits(dequantize(q, scales))


def _per_group_transpose(w, groups):
    """[G * N, K] -> [G * K, N]: each group's matrix transposed in place."""
    w = np.asarray(w, dtype=np.float64)
    N = w.shape[0] // groups
    return np.concatenate([w[g * N:(g + 1) * N].T for g in range(groups)])


def backward_bf16(x, w, dy, offs, groups):
    """Both gradients of Y = X W_g^T from float64 operands (bf16 values):
    dX = dY W_g per row group, dW_g = dY_g^T X_g. w is [G * N, K]."""
    dx = grouped_mm(dy, _per_group_transpose(w, groups), offs, groups)
    dw = grouped_mm_wgrad(np.asarray(dy, dtype=np.float64).T, np.asarray(x, dtype=np.float64).T, offs, groups)
    return dx, dw


def backward_high_precision(x_bits, w_bits, dy_bits, offs, groups):
    """The high-precision arm: the saved bf16 input and weight, unquantized."""
    return backward_bf16(bf16_to_f64(x_bits), bf16_to_f64(w_bits), bf16_to_f64(dy_bits), offs, groups)


def backward_dequantized(x_q, x_s, w_q, w_s, dy_bits, offs, groups):
    """The dequantized arm: the forward's dim0 codes of X [M, K] and W [G * N, K]
    (logical scales) dequantized to bf16; grad_out stays bf16."""
    xd = bf16_to_f64(dequantize_to_bf16_bits(x_q, x_s))
    wd = bf16_to_f64(dequantize_to_bf16_bits(w_q, w_s))
    return backward_bf16(xd, wd, bf16_to_f64(dy_bits), offs, groups)


# --------------------------------------------------------------------------------------
# Token-group padding (group sizes that are not multiples of 32)
# --------------------------------------------------------------------------------------
#
# The MoE stack pads each expert's token group to a multiple of the 32-row block
# before the grouped GEMM and unpads the outputs afterwards (pytorch/ao PR 4705,
# ghstack list: pad/unpad kernels; ao fork PR 10, "Known follow-ups": padded token
# groups for the grouped mm feed padded offsets to the GEMM). The pages print no
# layout. Reading taken here: group g's rows keep their order and move to a run
# that starts at the padded offset of g, the padded offsets being the running sum
# of the group sizes rounded up to 32; every other row of the padded buffer is
# zero. The buffer has a size fixed by (rows, groups) alone, so that no device
# value decides an allocation (rows + 31 * groups rounded up to 256); rows after
# the last padded offset belong to no group.


def padded_rows(rows, groups):
    """Rows of the padded buffer for any `groups` sizes summing to at most `rows`.

    A group grows by at most 31 rows, so rows + 31 * groups always suffices; the
    count is rounded up to a multiple of 256 so that the token axis, which becomes
    the row pitch of the transposed (dim1) codes, keeps whole 256-byte rows.
    """
    return -(-(rows + 31 * groups) // 256) * 256


def padded_offsets(offs):
    """offs_pad[g] = sum over j <= g of (size of group j rounded up to 32)."""
    out = []
    total = 0
    for start, end in group_bounds(offs, None):
        size = end - start
        total += ((size + 31) // 32) * 32
        out.append(total)
    return out


def pad_token_groups(x, offs, rows_pad):
    """x_pad [rows_pad, C]: row offs_pad[g-1] + i = row offs[g-1] + i of x for
    i < size of group g; all other rows zero. Returns (x_pad, offs_pad)."""
    x = np.asarray(x)
    pad_ends = padded_offsets(offs)
    out = np.zeros((rows_pad,) + x.shape[1:], dtype=x.dtype)
    pad_start = 0
    for (start, end), pad_end in zip(group_bounds(offs, None), pad_ends):
        for i in range(end - start):
            out[pad_start + i] = x[start + i]
        pad_start = pad_end
    return out, pad_ends


def unpad_token_groups(y_pad, offs, rows):
    """Inverse gather: row offs[g-1] + i of the result = row offs_pad[g-1] + i of
    y_pad. Rows past offs[G-1] belong to no group and stay zero."""
    y_pad = np.asarray(y_pad)
    pad_ends = padded_offsets(offs)
    out = np.zeros((rows,) + y_pad.shape[1:], dtype=y_pad.dtype)
    pad_start = 0
    for (start, end), pad_end in zip(group_bounds(offs, None), pad_ends):
        for i in range(end - start):
            out[start + i] = y_pad[pad_start + i]
        pad_start = pad_end
    return out


# --------------------------------------------------------------------------------------
# Output rounding and comparison metrics
# --------------------------------------------------------------------------------------


def round_to_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_to_bf16_bits(x):
    """Round float64 values to bf16 (round-to-nearest-even), returning uint16 patterns.

    Done directly from float64 (no intermediate float32, which could double-round):
    bf16 keeps 8 significant bits for normal values and a fixed 2^-133 grid below
    2^-126.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)  # a = f * 2^e, f in [0.5, 1)
    q_exp = np.maximum(e - 8, -133)  # grid spacing exponent
    out = np.ldexp(np.rint(np.ldexp(a, -q_exp)), q_exp)  # rint is round-half-even
    out = np.where(a == 0, 0.0, out)
    out = np.copysign(out, x)
    with np.errstate(over="ignore"):  # values at or above 2^128 become inf just below
        f32 = out.astype(np.float32)  # exact: out has <= 8 significant bits
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.abs(out) >= 2.0**128, (bits & 0x8000) | 0x7F80, bits)
    return bits.astype(np.uint16)


def rel_frobenius(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def bf16_ordinal(bits):
    """Map bf16 patterns to integers ordered like their values (for ulp distances)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def sqnr_db(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(10.0 * np.log10(np.sum(ref**2) / np.sum((ref - out) ** 2)))
