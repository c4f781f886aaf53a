// Token-group padding for the grouped GEMM (pytorch/ao PR 4705, ghstack list:
// pad/unpad kernels; ao fork PR 10, "Known follow-ups": padded token groups feed
// padded offsets to the grouped GEMM).
//
// Group g's rows [offs[g-1], offs[g]) move, in order, to the run starting at
// offs_pad[g-1], where offs_pad is the running sum of the group sizes rounded up
// to 32; every other row of the padded buffer is zero. Unpadding gathers the
// rows back. Both are pure row moves bound by HBM: 2 B read + 2 B written per
// real element and 2 B written per pad element (pad); element size read and
// written per grouped element (unpad).
//
// Every workgroup first rebuilds the group table in LDS from offs (G <= 1024
// int32, one wave, two 64-wide scans per 64 groups), so no second launch or
// device-wide barrier is needed, then its waves walk rows: one wave per row,
// 16-byte lanes, four loads in flight per lane before the stores. offs is
// sanitised while it is read (each end clamped into [0, rows] and made
// non-decreasing): an out-of-contract offs moves the wrong rows but never
// addresses memory outside the buffers.

#include "group_table.h"

namespace mx {

constexpr int kPadThreads = 256;

// Copies (src != nullptr) or zero-fills one row of `chunks` 16-byte chunks, one
// wave, four chunks per lane in flight.
__device__ inline void move_row(const u32x4* src, u32x4* dst, int64_t chunks, int lane) {
  for (int64_t c0 = 0; c0 < chunks; c0 += 256) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = c0 + 64 * j + lane;
      v[j] = (u32x4){0, 0, 0, 0};
      if (src && c < chunks) v[j] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = c0 + 64 * j + lane;
      if (c < chunks) dst[c] = v[j];
    }
  }
}

// x [rows x cols] bf16 (pitch ld_x) -> x_pad [rows_pad x cols] (pitch cols); block
// 0 also writes offs_pad.
__global__ __launch_bounds__(kPadThreads) void k_pad_rows(const uint16_t* __restrict__ x, int32_t rows, int64_t cols,
                                                          int64_t ld_x, const int32_t* __restrict__ offs, int groups,
                                                          uint16_t* __restrict__ x_pad, int64_t rows_pad,
                                                          int32_t* __restrict__ offs_pad) {
  __shared__ GroupTable t;
  build_table(t, offs, groups, rows);
  if (blockIdx.x == 0)
    for (int g = threadIdx.x; g < groups; g += kPadThreads) offs_pad[g] = t.pad_end[g];
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kPadThreads / 64);
  const int64_t chunks = cols / 8;
  for (int64_t p = (int64_t)blockIdx.x * (kPadThreads / 64) + (threadIdx.x >> 6); p < rows_pad; p += waves) {
    const int64_t s = padded_source(t, groups, p);
    move_row(s >= 0 ? (const u32x4*)(x + s * ld_x) : nullptr, (u32x4*)(x_pad + p * cols), chunks, lane);
  }
}

// y_pad [rows_pad x row_bytes] (pitch ld_pad bytes) -> y [rows x row_bytes] (pitch
// ld_y bytes) for the rows of every group; rows past the last group untouched.
__global__ __launch_bounds__(kPadThreads) void k_unpad_rows(const uint8_t* __restrict__ y_pad, int64_t rows_pad,
                                                            int64_t row_bytes, int64_t ld_pad,
                                                            const int32_t* __restrict__ offs, int groups,
                                                            uint8_t* __restrict__ y, int32_t rows, int64_t ld_y) {
  __shared__ GroupTable t;
  build_table(t, offs, groups, rows);
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kPadThreads / 64);
  const int64_t chunks = row_bytes / 16;
  const int64_t grouped = t.end[groups - 1];
  for (int64_t r = (int64_t)blockIdx.x * (kPadThreads / 64) + (threadIdx.x >> 6); r < grouped; r += waves) {
    const int g = upper_index(t.end, groups, r);  // < groups because r < end[groups-1]
    const int64_t src = (g ? t.pad_end[g - 1] : 0) + (r - (g ? t.end[g - 1] : 0));
    if (src >= rows_pad) continue;  // unreachable when rows_pad >= the padded size bound
    move_row((const u32x4*)(y_pad + src * ld_pad), (u32x4*)(y + r * ld_y), chunks, lane);
  }
}

// Checks offs against the grouped calls' preconditions. One workgroup: each thread
// tests its groups' ends against the previous end, the required multiple and
// [0, m]; the violation bits and the first offending group are reduced in LDS and
// written by thread 0 (no global atomics, nothing read back on the host).
__global__ __launch_bounds__(kPadThreads) void k_check_offs(const int32_t* __restrict__ offs, int groups, int64_t m,
                                                            int multiple, int32_t* __restrict__ result) {
  __shared__ int s_bits, s_first;
  if (threadIdx.x == 0) {
    s_bits = 0;
    s_first = 0x7FFFFFFF;
  }
  __syncthreads();
  int bits = 0, first = 0x7FFFFFFF;
  for (int g = threadIdx.x; g < groups; g += kPadThreads) {
    const int64_t e = offs[g], prev = g ? offs[g - 1] : 0;
    int b = 0;
    if (e < prev) b |= 1;                // decreasing
    if (e % multiple != 0) b |= 2;       // not a multiple
    if (e < 0 || e > m) b |= 4;          // outside [0, m]
    if (b) {
      bits |= b;
      first = g < first ? g : first;
    }
  }
  atomicOr(&s_bits, bits);
  atomicMin(&s_first, first);
  __syncthreads();
  if (threadIdx.x == 0) {
    result[0] = s_bits;
    result[1] = s_first == 0x7FFFFFFF ? -1 : s_first;
  }
}

// Workgroups: enough waves for every row, at most 8 workgroups per compute unit.
inline unsigned pad_grid(int64_t rows) {
  const int64_t need = (rows + kPadThreads / 64 - 1) / (kPadThreads / 64);
  const int64_t cap = 256 * 8;
  return (unsigned)(need < 1 ? 1 : (need < cap ? need : cap));
}

}  // namespace mx

hipError_t mx_launch_pad(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const int32_t* offs,
                         int groups, uint16_t* x_pad, int64_t rows_pad, int32_t* offs_pad, hipStream_t stream) {
  hipLaunchKernelGGL(mx::k_pad_rows, dim3(mx::pad_grid(rows_pad)), dim3(mx::kPadThreads), 0, stream, x, (int32_t)rows,
                     cols, ld_x, offs, groups, x_pad, rows_pad, offs_pad);
  return hipGetLastError();
}

hipError_t mx_launch_unpad(const void* y_pad, int64_t rows_pad, int64_t row_bytes, int64_t ld_pad_bytes,
                           const int32_t* offs, int groups, void* y, int64_t rows, int64_t ld_y_bytes,
                           hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(mx::k_unpad_rows, dim3(mx::pad_grid(rows)), dim3(mx::kPadThreads), 0, stream,
                     (const uint8_t*)y_pad, rows_pad, row_bytes, ld_pad_bytes, offs, groups, (uint8_t*)y,
                     (int32_t)rows, ld_y_bytes);
  return hipGetLastError();
}

hipError_t mx_launch_check_offs(const int32_t* offs, int groups, int64_t m, int multiple, int32_t* result,
                                hipStream_t stream) {
  hipLaunchKernelGGL(mx::k_check_offs, dim3(1), dim3(mx::kPadThreads), 0, stream, offs, groups, m, multiple, result);
  return hipGetLastError();
}
