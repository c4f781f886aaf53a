// Register-only loop of the block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4):
// the practical MXFP8 ceiling of the part, against which the GEMMs' rates are
// reported beside the nominal peak. The operands are fixed pseudo-random E4M3 codes
// (no NaN: the exponent's low bit cleared) with unit scales; each wave keeps four
// independent accumulation chains so the matrix core never waits on a result.
// 512 workgroups of four waves: two waves per SIMD on every compute unit.

#include "common.h"

namespace mx {

constexpr int kProbeBlocks = 512, kProbeThreads = 256, kProbeChains = 4;

__global__ __launch_bounds__(kProbeThreads) void k_mfma_probe(int64_t iters, float* __restrict__ sink) {
  v8i a, b;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    unsigned h = threadIdx.x * 0x9E3779B1u ^ (unsigned)d * 0x85EBCA77u ^ blockIdx.x * 0xC2B2AE3Du;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    a[d] = (int)(h & 0xF7F7F7F7u);
    b[d] = (int)((h * 0x27D4EB2Fu) & 0xF7F7F7F7u);
  }
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[threadIdx.x] = s;  // keeps the loop; every workgroup writes the same 256 floats
}

}  // namespace mx

// iters * 2^30 flops: 512 x 4 waves x 4 chains x iters MFMAs of 2 x 32 x 32 x 64.
hipError_t mx_launch_probe_mfma(int64_t iters, float* sink, hipStream_t stream) {
  static_assert(mx::kProbeBlocks * (mx::kProbeThreads / 64) * mx::kProbeChains * 2 * 32 * 32 * 64 == (1 << 30), "");
  hipLaunchKernelGGL(mx::k_mfma_probe, dim3(mx::kProbeBlocks), dim3(mx::kProbeThreads), 0, stream, iters, sink);
  return hipGetLastError();
}

// One block-scaled MFMA of either full-rate form on logical operands, for the
// numerics tests: a and b are row-major [R x K] E4M3 codes with row-major [R x K/32]
// E8M0 bytes; the single wave builds the instruction's register images from them
// (layouts measured on gfx950):
//   32x32x64: lane l holds row l % 32, contraction bytes [16h, 16h+16) and
//             [32+16h, 32+16h+16), h = l / 32; the scale of row r, block b comes
//             from lane r + 32b; output lane l, register v = row 8(v/4) + 4h + v%4
//             of the first operand, column l % 32 of the second.
//   16x16x128: lane l holds row l % 16, contraction bytes [16h, 16h+16) and
//             [64+16h, 64+16h+16), h = l / 16; the scale of row r, block b comes
//             from lane r + 16b; output lane l, register v = row 4h + v of the
//             first operand, column l % 16 of the second.
// `swap` passes b as the instruction's first operand (the order the GEMM uses) and
// transposes the result back, so d[i][j] always pairs row i of a with row j of b.
namespace mx {

template <int R, int K>
__device__ inline void probe_operand(const uint8_t* x, const uint8_t* xs, int l, v8i& reg, int& sc) {
  const int r = l % R, h = l / R;
  const uint8_t* row = x + r * K;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int k0 = d < 4 ? 16 * h + 4 * d : K / 2 + 16 * h + 4 * (d - 4);
    reg[d] = (int)((unsigned)row[k0] | (unsigned)row[k0 + 1] << 8 | (unsigned)row[k0 + 2] << 16 |
                   (unsigned)row[k0 + 3] << 24);
  }
  sc = xs[r * (K / 32) + h];
}

__global__ __launch_bounds__(64) void k_probe_dot(int form, const uint8_t* __restrict__ a,
                                                  const uint8_t* __restrict__ a_s, const uint8_t* __restrict__ b,
                                                  const uint8_t* __restrict__ b_s, const float* __restrict__ c,
                                                  float* __restrict__ d) {
  const int l = threadIdx.x;
  const bool swap = form & 2;
  if ((form & 1) == 0) {
    v8i ra, rb;
    int sa, sb;
    probe_operand<32, 64>(a, a_s, l, ra, sa);
    probe_operand<32, 64>(b, b_s, l, rb, sb);
    v16f acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v / 4) + 4 * (l / 32) + v % 4, col = l % 32;
      acc[v] = swap ? c[col * 32 + r] : c[r * 32 + col];
    }
    acc = swap ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(rb, ra, acc, 0, 0, 0, sb, 0, sa)
               : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ra, rb, acc, 0, 0, 0, sa, 0, sb);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v / 4) + 4 * (l / 32) + v % 4, col = l % 32;
      d[swap ? col * 32 + r : r * 32 + col] = acc[v];
    }
  } else {
    v8i ra, rb;
    int sa, sb;
    probe_operand<16, 128>(a, a_s, l, ra, sa);
    probe_operand<16, 128>(b, b_s, l, rb, sb);
    v4f acc;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 4 * (l / 16) + v, col = l % 16;
      acc[v] = swap ? c[col * 16 + r] : c[r * 16 + col];
    }
    acc = swap ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rb, ra, acc, 0, 0, 0, sb, 0, sa)
               : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ra, rb, acc, 0, 0, 0, sa, 0, sb);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 4 * (l / 16) + v, col = l % 16;
      d[swap ? col * 16 + r : r * 16 + col] = acc[v];
    }
  }
}

}  // namespace mx

hipError_t mx_launch_probe_dot(int form, const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                               const float* c, float* d, hipStream_t stream) {
  hipLaunchKernelGGL(mx::k_probe_dot, dim3(1), dim3(64), 0, stream, form, a, a_s, b, b_s, c, d);
  return hipGetLastError();
}
