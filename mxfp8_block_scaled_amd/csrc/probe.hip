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
