// Internal helpers shared by the cast and GEMM kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// MFMA-blocked scale layout: tiles of 32 rows x 8 blocks (256 B), row-band major.
__host__ __device__ inline int64_t scale_tiles_k(int64_t kb) { return (kb + 7) / 8; }

__host__ __device__ inline int64_t scale_tile_base(int64_t row_band, int64_t kt, int64_t tiles_k) {
  return (row_band * tiles_k + kt) * 256;
}

// Byte position of block kb (0..7 within its tile) of row r (0..31 within the band).
__host__ __device__ inline int scale_in_tile(int r, int kb) { return (kb & 1) * 128 + r * 4 + ((kb & 7) >> 1); }

// RCEIL E8M0 byte from the bf16 bits of a block amax (sign already cleared).
// amax = (1 + m/128) * 2^(E-127); ceil(log2(amax/448)) = E - 135 + [m > 96]
// because 448 = 1.75 * 2^8 and 1 + 96/128 = 1.75. Zero, bf16-denormal and tiny
// amax clamp to byte 0. Finite input never reaches the upper clamp (max 247).
__device__ inline int rceil_byte(unsigned amax_bits) {
  int e = (int)(amax_bits >> 7);
  int b = e - 8 + ((amax_bits & 0x7f) > 0x60 ? 1 : 0);
  b = e == 0 ? 0 : b;
  return b < 0 ? 0 : b;
}

// FLOOR E8M0 byte (the OCP MX default): floor(log2(amax)) - 8 = E - 135 for bf16
// exponent field E >= 1, so the byte is E - 8, clamped at 0 (zero and bf16-denormal
// amax included).
__device__ inline int floor_byte(unsigned amax_bits) {
  int b = (int)(amax_bits >> 7) - 8;
  return b < 0 ? 0 : b;
}

template <bool FLOOR>
__device__ inline int scale_byte(unsigned amax_bits) {
  return FLOOR ? floor_byte(amax_bits) : rceil_byte(amax_bits);
}

// E8M0 byte as the float operand of the scaled converts: only the exponent
// field is used, so the bits are just byte << 23.
__device__ inline float scale_operand(int byte) { return __builtin_bit_cast(float, (unsigned)byte << 23); }

// Encode two bf16 values (packed in one dword) as two E4M3 codes (low 16 bits of
// the result) = RNE E4M3 of x / 2^(byte - 127). A quotient that rounds above 448
// comes out as NaN (S.1111.111), not saturated: the RCEIL rule never produces one,
// the FLOOR rule does and fixes the codes with sat_e4m3x4. `byte` must be >= 1
// here; blocks whose scale byte is 0 are handled by the callers by doubling the
// input and using byte 1 (exact: x / 2^-127 == 2x / 2^-126).
__device__ inline unsigned cvt2(unsigned two_bf16, float scale) {
  bf16x2 v = __builtin_bit_cast(bf16x2, two_bf16);
  s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16((s16x2){0, 0}, v, scale, false);
  return (unsigned)(unsigned short)r[0];
}

// Saturates four packed E4M3 codes: a NaN byte (S.1111.111), which from finite
// input only the convert's overflow produces, becomes +-448 (S.1111.110). The low
// seven bits of a byte plus one carry into its bit 7 exactly when they are all ones,
// and never into the next byte.
__device__ inline unsigned sat_e4m3x4(unsigned d) {
  return d ^ ((((d & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u) >> 7);
}

// Doubles two packed bf16 values exactly, for |x| tiny (both inputs well below
// 2^126): a bf16-denormal doubles by shifting its magnitude bits, a normal value
// by adding one to its exponent field.
__device__ inline unsigned double_bf16x2(unsigned v) {
  unsigned out = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    unsigned x = (v >> (16 * h)) & 0xffff;
    unsigned mag = x & 0x7fff;
    unsigned d = (mag & 0x7f80) == 0 ? (mag << 1) : (mag + 0x80);
    out |= ((x & 0x8000) | d) << (16 * h);
  }
  return out;
}

// max over the two bf16 magnitudes packed in a dword (as unsigned 16-bit values)
__device__ inline unsigned amax_pair(unsigned acc, unsigned v) {
  u16x2 a = __builtin_bit_cast(u16x2, acc);
  u16x2 b = __builtin_bit_cast(u16x2, v & 0x7fff7fffu);
  return __builtin_bit_cast(unsigned, __builtin_elementwise_max(a, b));
}

__device__ inline unsigned fold_pair(unsigned acc) {
  unsigned lo = acc & 0xffff, hi = acc >> 16;
  return lo > hi ? lo : hi;
}

// DPP quad permutations: lane i takes the value of lane (i ^ 1) / (i ^ 2) of its quad.
__device__ inline unsigned dpp_xor1(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ inline unsigned dpp_xor2(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}

__device__ inline unsigned umax(unsigned a, unsigned b) { return a > b ? a : b; }

// Two floats -> two bf16 (round to nearest even; NaN stays NaN), packed a | b << 16:
// one v_cvt_pk_bf16_f32.
__device__ inline unsigned bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((v2f){a, b}, bf16x2));
}

}  // namespace mx
