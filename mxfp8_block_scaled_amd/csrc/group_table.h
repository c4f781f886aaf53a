// Token-group table shared by the padding kernels and the padded cast: group ends
// and padded group ends (each group's row count rounded up to 32), rebuilt in LDS by
// every workgroup from the device offs (ao fork PR 10, "Known follow-ups": padded
// token groups; pytorch/ao PR 4705, ghstack list: pad/unpad kernels).
#pragma once

#include "common.h"

namespace mx {

constexpr int kPadMaxGroups = 1024;

struct GroupTable {
  int32_t end[kPadMaxGroups];      // sanitised group ends (unpadded rows)
  int32_t pad_end[kPadMaxGroups];  // padded group ends
};

// Fills the table (wave 0) and synchronises the workgroup. rows <= 2^31 - 1 and
// the padded total <= rows + 31 * groups < 2^31 (checked on the host).
__device__ inline void build_table(GroupTable& t, const int32_t* offs, int groups, int32_t rows) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int32_t carry_end = 0, carry_pad = 0;
    for (int g0 = 0; g0 < groups; g0 += 64) {
      const int g = g0 + lane;
      int32_t e = g < groups ? offs[g] : rows;
      e = e < 0 ? 0 : (e > rows ? rows : e);
      // inclusive prefix max: the sanitised ends
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int32_t u = __shfl_up(e, d);
        if (lane >= d) e = e > u ? e : u;
      }
      e = e > carry_end ? e : carry_end;
      int32_t prev = __shfl_up(e, 1);
      if (lane == 0) prev = carry_end;
      int32_t p = ((e - prev) + 31) & ~31;  // padded size of the group
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int32_t u = __shfl_up(p, d);
        if (lane >= d) p += u;
      }
      p += carry_pad;
      if (g < groups) {
        t.end[g] = e;
        t.pad_end[g] = p;
      }
      carry_end = __shfl(e, 63);
      carry_pad = __shfl(p, 63);
    }
  }
  __syncthreads();
}

// First index g in [0, n) with v[g] > x, or n.
__device__ inline int upper_index(const int32_t* v, int n, int64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)v[mid] > x) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Source row of padded row p: the row of x it holds, or -1 for a padding row or a
// row past the last group.
__device__ inline int64_t padded_source(const GroupTable& t, int groups, int64_t p) {
  const int g = upper_index(t.pad_end, groups, p);
  if (g >= groups) return -1;
  const int64_t start = g ? t.end[g - 1] : 0;
  const int64_t i = p - (g ? t.pad_end[g - 1] : 0);
  return i < t.end[g] - start ? start + i : -1;
}

}  // namespace mx
