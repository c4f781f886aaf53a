// Conversions for the backward override arms (ao fork PR 10, "Design notes": the
// dequantized arm dequantizes the saved quantized forward operands for bf16 grouped
// GEMMs, and needs the scales in their logical, pre-blocking order; the
// high-precision arm runs the same GEMMs on the saved bf16 operands).
//
//   k_dequant      E4M3 codes + MFMA-blocked E8M0 scales -> bf16, same orientation
//                  (also the first step of the GEMMs computed from codes on the bf16 MFMA)
//   k_tile_t<IN>   transposes [rows x cols] tiles of bf16 (IN_BF16) or of codes
//                  dequantized on the way (IN_MXFP8) into bf16 [cols x rows], so
//                  the GEMM reads every operand contraction-contiguous
//   k_scales_logical  MFMA-blocked scale bytes -> logical [rows x cols/32]
//
// All are bound by HBM. The dequantized value code * 2^(byte - 127) is built in
// bf16's fields with integer operations: it is exact unless it falls below 2^-126
// (rounded to nearest even on bf16's 2^-133 grid) or reaches 2^128 (infinity), so no
// fp32 flush-to-zero mode can change a result.

#include <type_traits>

#include "common.h"

namespace mx {

// bf16 bits of value(code) * 2^(byte - 127), round-to-nearest-even.
__device__ inline unsigned deq_bf16(unsigned code, int byte) {
  const unsigned sign = (code & 0x80) << 8;
  const int e = (int)((code >> 3) & 15), m = (int)(code & 7);
  if ((code & 0x7F) == 0x7F) return sign | 0x7FC0;  // NaN code
  if (e == 0 && m == 0) return sign;
  // value = f * 2^(x - 3) with f in [8, 16)
  int f, x;
  if (e == 0) {  // E4M3 subnormal m * 2^-9: normalise m (1..7) into [8, 16)
    const int lz = m >= 4 ? 1 : (m >= 2 ? 2 : 3);
    f = m << lz;
    x = -6 - lz;
  } else {
    f = 8 + m;
    x = e - 7;
  }
  x += byte - 127;
  const int biased = x + 127;
  if (biased >= 255) return sign | 0x7F80;
  if (biased >= 1) return sign | ((unsigned)biased << 7) | ((unsigned)(f - 8) << 4);
  // bf16 subnormal: value / 2^-133 = f * 2^(x + 130), x + 130 <= 3
  const int sh = x + 130;
  unsigned q;
  if (sh >= 0) {
    q = (unsigned)f << sh;
  } else {
    const int k = -sh;
    if (k > 5) return sign;  // f < 16 <= 2^(k-1): below half of 2^-133
    q = (unsigned)f >> k;
    const unsigned r = (unsigned)f & ((1u << k) - 1), half = 1u << (k - 1);
    if (r > half || (r == half && (q & 1))) ++q;
  }
  return sign | q;
}

__device__ inline int scale_at(const uint8_t* scale, int64_t row, int64_t kb, int64_t kt) {
  return scale[scale_tile_base(row / 32, kb / 8, kt) + scale_in_tile((int)(row & 31), (int)(kb & 7))];
}

// deq_bf16 for scale bytes 10..246, where every non-zero code lands in bf16's normal
// range (the smallest, 2^-9, has exponent field byte - 9 >= 1; the largest, 448, has
// byte + 8 <= 254): the fields are placed directly, with selects instead of branches.
__device__ inline unsigned deq_bf16_normal(unsigned code, int byte) {
  const unsigned sign = (code & 0x80) << 8;
  const unsigned e = (code >> 3) & 15, m = code & 7;
  const unsigned lz = m >= 4 ? 1 : (m >= 2 ? 2 : 3);  // E4M3 subnormal m 2^-9 = (m << lz) 2^(-9-lz)
  const unsigned normal = ((e + (unsigned)byte - 7) << 7) | (m << 4);
  const unsigned subnormal = (((unsigned)byte - 6 - lz) << 7) | (((m << lz) - 8) << 4);
  unsigned bits = e ? normal : subnormal;
  bits = (code & 0x7f) == 0 ? 0u : bits;
  bits = (code & 0x7f) == 0x7f ? 0x7FC0u : bits;
  return sign | bits;
}

// 16 codes (one half-block) -> 16 bf16 in eight dwords
__device__ inline void deq16(u32x4 c, int byte, unsigned out[8]) {
  const unsigned w[4] = {c.x, c.y, c.z, c.w};
  if (byte >= 10 && byte <= 246) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      out[2 * d] = deq_bf16_normal(w[d] & 0xff, byte) | (deq_bf16_normal((w[d] >> 8) & 0xff, byte) << 16);
      out[2 * d + 1] = deq_bf16_normal((w[d] >> 16) & 0xff, byte) | (deq_bf16_normal(w[d] >> 24, byte) << 16);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      out[2 * d] = deq_bf16(w[d] & 0xff, byte) | (deq_bf16((w[d] >> 8) & 0xff, byte) << 16);
      out[2 * d + 1] = deq_bf16((w[d] >> 16) & 0xff, byte) | (deq_bf16(w[d] >> 24, byte) << 16);
    }
  }
}

// q [rows x cols] (pitch cols) -> out [rows x cols] bf16 (pitch cols). Each thread takes
// four chunks of 16 codes per pass, 256 chunks apart, so each load instruction of a wave
// reads 1 KB of consecutive codes and a thread has four loads in flight before it converts;
// chunk indexes are 32-bit below 2^31 chunks (WIDE: 64-bit beyond).
template <bool WIDE>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ scale,
                                                 int64_t rows, int64_t cols, uint16_t* __restrict__ out) {
  using I = std::conditional_t<WIDE, int64_t, uint32_t>;
  constexpr int U = 4;
  const I per_row = (I)(cols / 16), n = (I)(rows * (cols / 16));
  const int64_t kt = scale_tiles_k(cols / 32);
  const I step = (I)gridDim.x * (256 * U);
  for (I i0 = (I)blockIdx.x * (256 * U) + (I)threadIdx.x; i0 < n; i0 += step) {
    u32x4 codes[U];
    int byte[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const I i = i0 + (I)(256 * k);
      codes[k] = (u32x4){0, 0, 0, 0};
      byte[k] = 127;
      if (i < n) {
        const I r = i / per_row;
        codes[k] = __builtin_nontemporal_load((const u32x4*)(q + (int64_t)i * 16));
        byte[k] = scale_at(scale, (int64_t)r, (int64_t)((i - r * per_row) / 2), kt);
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const I i = i0 + (I)(256 * k);
      if (i < n) {
        unsigned o[8];
        deq16(codes[k], byte[k], o);
        u32x4* dst = (u32x4*)(out + (int64_t)i * 16);
        dst[0] = (u32x4){o[0], o[1], o[2], o[3]};
        dst[1] = (u32x4){o[4], o[5], o[6], o[7]};
      }
    }
  }
}

enum { IN_BF16 = 0, IN_MXFP8 = 1 };
constexpr int kT = 64;  // tile rows (elements)
// tile columns: 64 for bf16 input; 128 for codes, so that each thread moves two 16-byte
// chunks of codes (more bytes in flight per workgroup)
template <int IN>
constexpr int tile_cols() { return IN == IN_BF16 ? 64 : 128; }

// One 64 x TC tile per workgroup (256 threads): rows [r0, r0+64) x cols [c0, c0+TC)
// of batch b of `in` go to rows [c0, c0+TC) x cols [r0, r0+64) of batch b of `out`.
// The input is read as whole 16-byte chunks, staged in LDS row by row (padded pitch),
// and written as 16-byte chunks of the transposed rows. Ragged edges: rows and
// columns past the matrix are skipped (cols % 8 == 0, rows % 8 == 0 for bf16 input;
// cols % 32 == 0 for codes).
template <int IN>
__global__ __launch_bounds__(256) void k_tile_t(const void* __restrict__ in, const uint8_t* __restrict__ scale,
                                                int64_t rows, int64_t cols, int64_t ld_in, int64_t tiles_r,
                                                int64_t tiles_c, uint16_t* __restrict__ out) {
  constexpr int TC = tile_cols<IN>();
  constexpr int TP = TC + 2;  // LDS row pitch in bf16 (an odd number of 4-byte banks)
  __shared__ uint16_t t[kT * TP];
  const int tid = threadIdx.x;
  const int64_t per_batch = tiles_r * tiles_c;
  const int64_t b = blockIdx.x / per_batch, rest = blockIdx.x - b * per_batch;
  const int64_t r0 = (rest / tiles_c) * kT, c0 = (rest % tiles_c) * TC;
  if (IN == IN_BF16) {
    const uint16_t* x = (const uint16_t*)in + b * rows * ld_in;
#pragma unroll
    for (int k = 0; k < 2; ++k) {  // 64 rows x 8 chunks of 8 bf16
      const int id = tid + 256 * k, r = id >> 3, ch = id & 7;
      u32x4 v = (u32x4){0, 0, 0, 0};
      if (r0 + r < rows && c0 + 8 * ch < cols) v = __builtin_nontemporal_load((const u32x4*)(x + (r0 + r) * ld_in + c0 + 8 * ch));
      unsigned* dst = (unsigned*)(t + r * TP + 8 * ch);
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
  } else {
    const uint8_t* qb = (const uint8_t*)in + b * rows * ld_in;
    const int64_t kt = scale_tiles_k(cols / 32);
    u32x4 codes[2];
    int byte[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {  // 64 rows x 8 chunks of 16 codes: loads first, then the math
      const int id = tid + 256 * k, r = id >> 3, ch = id & 7;
      codes[k] = (u32x4){0, 0, 0, 0};
      byte[k] = 127;
      if (r0 + r < rows && c0 + 16 * ch < cols) {
        codes[k] = __builtin_nontemporal_load((const u32x4*)(qb + (r0 + r) * ld_in + c0 + 16 * ch));
        byte[k] = scale_at(scale, b * rows + r0 + r, (c0 + 16 * ch) / 32, kt);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int id = tid + 256 * k, r = id >> 3, ch = id & 7;
      unsigned o[8];
      deq16(codes[k], byte[k], o);
      unsigned* dst = (unsigned*)(t + r * TP + 16 * ch);
#pragma unroll
      for (int d = 0; d < 8; ++d) dst[d] = o[d];
    }
  }
  __syncthreads();
  uint16_t* ob = out + b * cols * rows;
#pragma unroll
  for (int k = 0; k < TC / 32; ++k) {  // TC output rows (input columns) x 8 chunks of 8 input rows
    const int id = tid + 256 * k, c = id >> 3, rc = id & 7;
    if (c0 + c >= cols || r0 + 8 * rc >= rows) continue;
    unsigned w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      w[d] = (unsigned)t[(8 * rc + 2 * d) * TP + c] | ((unsigned)t[(8 * rc + 2 * d + 1) * TP + c] << 16);
    *(u32x4*)(ob + (c0 + c) * rows + r0 + 8 * rc) = (u32x4){w[0], w[1], w[2], w[3]};
  }
}

// MFMA-blocked scales of [rows x cols] -> logical [rows x cols/32]; one byte per thread.
__global__ __launch_bounds__(256) void k_scales_logical(const uint8_t* __restrict__ scale, int64_t rows,
                                                        int64_t kb, uint8_t* __restrict__ logical) {
  const int64_t n = rows * kb, kt = scale_tiles_k(kb);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / kb, k = i - r * kb;
    logical[i] = (uint8_t)scale_at(scale, r, k, kt);
  }
}

inline unsigned grid_for(int64_t n_threads) {
  const int64_t b = (n_threads + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b < 256 * 16 ? b : 256 * 16));
}

}  // namespace mx

hipError_t mx_launch_dequant(const uint8_t* q, const uint8_t* scale, int64_t batch, int64_t rows, int64_t cols,
                             int transpose, uint16_t* out, hipStream_t stream) {
  if (batch * rows == 0) return hipSuccess;
  if (!transpose) {
    const int64_t chunks = batch * rows * cols / 16;
    const dim3 grid(mx::grid_for((chunks + 3) / 4));  // four chunks per thread and pass
    if (chunks < ((int64_t)1 << 31))
      hipLaunchKernelGGL(mx::k_dequant<false>, grid, dim3(256), 0, stream, q, scale, batch * rows, cols, out);
    else
      hipLaunchKernelGGL(mx::k_dequant<true>, grid, dim3(256), 0, stream, q, scale, batch * rows, cols, out);
  } else {
    constexpr int TC = mx::tile_cols<mx::IN_MXFP8>();
    const int64_t tr = (rows + mx::kT - 1) / mx::kT, tc = (cols + TC - 1) / TC;
    hipLaunchKernelGGL(mx::k_tile_t<mx::IN_MXFP8>, dim3((unsigned)(batch * tr * tc)), dim3(256), 0, stream,
                       (const void*)q, scale, rows, cols, cols, tr, tc, out);
  }
  return hipGetLastError();
}

hipError_t mx_launch_transpose_bf16(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                                    uint16_t* out, hipStream_t stream) {
  if (batch * rows == 0) return hipSuccess;
  constexpr int TC = mx::tile_cols<mx::IN_BF16>();
  const int64_t tr = (rows + mx::kT - 1) / mx::kT, tc = (cols + TC - 1) / TC;
  hipLaunchKernelGGL(mx::k_tile_t<mx::IN_BF16>, dim3((unsigned)(batch * tr * tc)), dim3(256), 0, stream,
                     (const void*)x, (const uint8_t*)nullptr, rows, cols, ld, tr, tc, out);
  return hipGetLastError();
}

hipError_t mx_launch_scales_logical(const uint8_t* scale, int64_t rows, int64_t cols, uint8_t* logical,
                                    hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(mx::k_scales_logical, dim3(mx::grid_for(rows * (cols / 32))), dim3(256), 0, stream, scale, rows,
                     cols / 32, logical);
  return hipGetLastError();
}
