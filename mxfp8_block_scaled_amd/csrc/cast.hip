// MXFP8 training casts for gfx950: dim0 (rowwise 1x32), dim1 (columnwise 32x1,
// written transposed) and the 32x32 weight form.
//
// Numerics (OCP MX): block amax of |x| taken as an unsigned max over the bf16 bit
// patterns with the sign cleared (monotone for finite values); RCEIL E8M0 byte from
// the amax bits by an integer closed form (no division, no log, so no fp32
// flush-to-zero hazard); elements encoded by the gfx950 scaled convert
// (v_cvt_scalef32_pk_fp8_bf16), which computes the RNE, saturating E4M3 code of
// x / 2^(byte-127) directly from bf16, two elements per instruction. Scales are
// written in the MFMA-blocked layout the grouped GEMM reads, so no rearrange pass
// follows (torchtitan PR 5334, body: blocked E8M0 scales emitted directly).

#include "common.h"

namespace mx {

// Encode 8 bf16 values (one 16-byte chunk) with scale byte `byte` of a block whose
// amax bits are `amax`: returns 8 codes in two dwords.
__device__ inline u32x2 encode8(u32x4 v, int byte, unsigned amax) {
  bool tiny = (byte == 0) && (amax != 0);
  float sc = scale_operand(byte == 0 ? 1 : byte);
  u32x2 out;
  if (tiny) {
    out.x = cvt2(double_bf16x2(v.x), sc) | (cvt2(double_bf16x2(v.y), sc) << 16);
    out.y = cvt2(double_bf16x2(v.z), sc) | (cvt2(double_bf16x2(v.w), sc) << 16);
  } else {
    out.x = cvt2(v.x, sc) | (cvt2(v.y, sc) << 16);
    out.y = cvt2(v.z, sc) | (cvt2(v.w, sc) << 16);
  }
  return out;
}

__device__ inline unsigned amax8(u32x4 v) {
  unsigned a = amax_pair(0u, v.x);
  a = amax_pair(a, v.y);
  a = amax_pair(a, v.z);
  a = amax_pair(a, v.w);
  return fold_pair(a);
}

// ---------------------------------------------------------------------------------
// dim0: one wave per 32-row x 256-column tile (exactly one 256-byte scale tile).
// Lane l reads 16-byte chunk (l % 32) of rows 2i + l/32, i = 0..15; the four lanes
// of a quad hold one 32-element block, reduced with two DPP quad permutes.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_dim0(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ld, uint8_t* __restrict__ q, uint8_t* __restrict__ scale,
                                                    int64_t row_bands, int64_t ktiles) {
  __shared__ unsigned s_tile[4][64];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, c = l & 31;
  const int64_t t = (int64_t)blockIdx.x * 4 + w;
  const bool active = t < row_bands * ktiles;
  const int64_t rb = active ? t / ktiles : 0, kt = active ? t % ktiles : 0;
  const int64_t col0 = kt * 256 + c * 8;
  const bool col_ok = active && col0 < cols;
  s_tile[w][l] = 0x7f7f7f7fu;
  __syncthreads();

  u32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int64_t r = rb * 32 + 2 * i + h;
    v[i] = (u32x4){0, 0, 0, 0};
    if (col_ok && r < rows) v[i] = *(const u32x4*)(x + r * ld + col0);
  }
  uint8_t* st = (uint8_t*)s_tile[w];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int64_t r = rb * 32 + 2 * i + h;
    unsigned a = amax8(v[i]);
    a = umax(a, dpp_xor1(a));
    a = umax(a, dpp_xor2(a));
    int byte = rceil_byte(a);
    u32x2 codes = encode8(v[i], byte, a);
    if (col_ok && r < rows) {
      *(u32x2*)(q + r * cols + col0) = codes;
      if ((c & 3) == 0) st[scale_in_tile(2 * i + h, c >> 2)] = (uint8_t)byte;
    }
  }
  __syncthreads();
  if (active) ((unsigned*)(scale + scale_tile_base(rb, kt, ktiles)))[l] = s_tile[w][l];
}

// ---------------------------------------------------------------------------------
// dim1: a workgroup covers 256 input rows x 128 input columns of one batch. Wave w
// takes rows 64w..64w+63; lane l takes the column pair (2l, 2l+1), one dword per
// row, so every load instruction reads 256 contiguous bytes. Each lane then owns
// two 32-row blocks of two columns and reduces them in registers; the codes of a
// block are 32 contiguous bytes of an output row of q_t.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_dim1(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ld, uint8_t* __restrict__ q_t,
                                                    uint8_t* __restrict__ scale_t, int64_t rtiles, int64_t ctiles) {
  __shared__ unsigned s_tiles[4][64];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t bid = blockIdx.x;
  const int64_t b = bid / (rtiles * ctiles);
  const int64_t rem = bid % (rtiles * ctiles);
  const int64_t ct = rem / rtiles, rt = rem % rtiles;
  const int64_t c = ct * 128 + 2 * l;
  const bool col_ok = c < cols;
  const uint16_t* xb = x + b * rows * ld;
  uint8_t* qb = q_t + b * cols * rows;
  s_tiles[w][l] = 0x7f7f7f7fu;
  __syncthreads();

  const int64_t r0 = rt * 256 + 64 * w;
  unsigned v[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    int64_t r = r0 + j;
    v[j] = 0;
    if (col_ok && r < rows) v[j] = *(const unsigned*)(xb + r * ld + c);
  }
  uint8_t* st = (uint8_t*)s_tiles;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int64_t rb = r0 + 32 * half;  // first input row of the block
    unsigned am = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) am = amax_pair(am, v[32 * half + j]);
    const unsigned a_lo = am & 0xffff, a_hi = am >> 16;
    const int b_lo = rceil_byte(a_lo), b_hi = rceil_byte(a_hi);
    const bool tiny_lo = b_lo == 0 && a_lo != 0, tiny_hi = b_hi == 0 && a_hi != 0;
    const float s_lo = scale_operand(b_lo == 0 ? 1 : b_lo), s_hi = scale_operand(b_hi == 0 ? 1 : b_hi);
    unsigned o_lo[8], o_hi[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      unsigned cl[2], ch[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const unsigned v0 = v[32 * half + 4 * p + 2 * e], v1 = v[32 * half + 4 * p + 2 * e + 1];
        unsigned lo = __builtin_amdgcn_perm(v1, v0, 0x05040100u);  // (col lo of row j, col lo of row j+1)
        unsigned hi = __builtin_amdgcn_perm(v1, v0, 0x07060302u);  // (col hi of row j, col hi of row j+1)
        if (tiny_lo) lo = double_bf16x2(lo);
        if (tiny_hi) hi = double_bf16x2(hi);
        cl[e] = cvt2(lo, s_lo);
        ch[e] = cvt2(hi, s_hi);
      }
      o_lo[p] = cl[0] | (cl[1] << 16);
      o_hi[p] = ch[0] | (ch[1] << 16);
    }
    if (col_ok && rb < rows) {
      u32x4* d0 = (u32x4*)(qb + c * rows + rb);
      u32x4* d1 = (u32x4*)(qb + (c + 1) * rows + rb);
      d0[0] = (u32x4){o_lo[0], o_lo[1], o_lo[2], o_lo[3]};
      d0[1] = (u32x4){o_lo[4], o_lo[5], o_lo[6], o_lo[7]};
      d1[0] = (u32x4){o_hi[0], o_hi[1], o_hi[2], o_hi[3]};
      d1[1] = (u32x4){o_hi[4], o_hi[5], o_hi[6], o_hi[7]};
      // scale tile (l / 16) of this workgroup, rows 2l % 32 and (2l+1) % 32, block 2w + half
      const int tile = l >> 4, kb = 2 * w + half;
      st[tile * 256 + scale_in_tile((2 * l) & 31, kb)] = (uint8_t)b_lo;
      st[tile * 256 + scale_in_tile((2 * l + 1) & 31, kb)] = (uint8_t)b_hi;
    }
  }
  __syncthreads();
  // thread t writes dword t % 64 of scale tile t / 64
  const int tile = threadIdx.x >> 6;
  const int64_t out_row0 = ct * 128 + 32 * tile;  // first output row (input column) of the tile
  if (out_row0 < cols) {
    const int64_t band = (b * cols + out_row0) / 32;
    const int64_t ktiles = scale_tiles_k(rows / 32);
    ((unsigned*)(scale_t + scale_tile_base(band, rt, ktiles)))[l] = s_tiles[tile][l];
  }
}

// ---------------------------------------------------------------------------------
// 32x32 weight cast: one wave per 32-row x 256-column strip (eight 32x32 tiles).
// The tile amax reduces over the lane's 16 rows, the quad (32 columns) and the two
// wave halves. Codes go out rowwise directly and, through LDS, transposed.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_w32(const uint16_t* __restrict__ w, int64_t batch, int64_t n,
                                                   int64_t k, int64_t ld, uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ q_t, uint8_t* __restrict__ s_row,
                                                   uint8_t* __restrict__ s_col, int64_t ktiles) {
  __shared__ unsigned lds_q[4][32 * 64];  // per wave: 32 rows x 256 bytes
  __shared__ uint8_t lds_tb[4][8];
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, c = l & 31;
  const int64_t row_bands = batch * n / 32;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  const bool active = t < row_bands * ktiles;
  const int64_t rb = active ? t / ktiles : 0, kt = active ? t % ktiles : 0;
  const int64_t col0 = kt * 256 + c * 8;
  const bool col_ok = active && col0 < k;
  const int64_t kb_total = k / 32;

  u32x4 v[16];
  unsigned a = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int64_t r = rb * 32 + 2 * i + h;
    v[i] = (u32x4){0, 0, 0, 0};
    if (col_ok) v[i] = *(const u32x4*)(w + r * ld + col0);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) a = umax(a, amax8(v[i]));
  a = umax(a, dpp_xor1(a));
  a = umax(a, dpp_xor2(a));
  a = umax(a, (unsigned)__shfl_xor((int)a, 32));
  const int byte = rceil_byte(a);
  if (h == 0 && (c & 3) == 0) lds_tb[wv][c >> 2] = (uint8_t)byte;

  uint8_t* lq = (uint8_t*)lds_q[wv];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int64_t r = rb * 32 + 2 * i + h;
    u32x2 codes = encode8(v[i], byte, a);
    if (col_ok) *(u32x2*)(q + r * k + col0) = codes;
    *(u32x2*)(lq + (2 * i + h) * 256 + c * 8) = codes;
  }
  __syncthreads();
  if (!active) return;
  // rowwise scales: lane l's dword = tile bytes of blocks h, 2+h, 4+h, 6+h for row l%32
  {
    unsigned d = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int kb = kt * 8 + 2 * j + h;
      unsigned bj = kb < kb_total ? lds_tb[wv][2 * j + h] : 0x7fu;
      d |= bj << (8 * j);
    }
    ((unsigned*)(s_row + scale_tile_base(rb, kt, ktiles)))[l] = d;
  }
  if (q_t == nullptr) return;
  // transposed codes: lane l writes output rows kk = kt*256 + 4l + j (j = 0..3),
  // columns rb_local*32 .. +31 of batch bi.
  const int64_t bi = (rb * 32) / n;
  const int64_t nb_local = (rb * 32 - bi * n) / 32;  // 32-column band of q_t within the batch
  if (kt * 256 + 4 * l >= k) return;
  unsigned outw[4][8];
#pragma unroll
  for (int a8 = 0; a8 < 8; ++a8) {
    unsigned d0 = lds_q[wv][(4 * a8 + 0) * 64 + l];
    unsigned d1 = lds_q[wv][(4 * a8 + 1) * 64 + l];
    unsigned d2 = lds_q[wv][(4 * a8 + 2) * 64 + l];
    unsigned d3 = lds_q[wv][(4 * a8 + 3) * 64 + l];
    unsigned t0 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
    unsigned t1 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
    unsigned t2 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
    unsigned t3 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
    outw[0][a8] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
    outw[1][a8] = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
    outw[2][a8] = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
    outw[3][a8] = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
  }
  uint8_t* qtb = q_t + bi * k * n;
  const unsigned tb = lds_tb[wv][l >> 3];
  const int64_t kt_col = nb_local / 8;
  const int64_t ktiles_col = scale_tiles_k(n / 32);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t kk = kt * 256 + 4 * l + j;
    u32x4* dst = (u32x4*)(qtb + kk * n + nb_local * 32);
    dst[0] = (u32x4){outw[j][0], outw[j][1], outw[j][2], outw[j][3]};
    dst[1] = (u32x4){outw[j][4], outw[j][5], outw[j][6], outw[j][7]};
    const int64_t band = (bi * k + kk) / 32;
    uint8_t* sc = s_col + scale_tile_base(band, kt_col, ktiles_col);
    sc[scale_in_tile((int)(kk & 31), (int)(nb_local & 7))] = (uint8_t)tb;
    // the last column band of the batch also fills the layout's pad blocks
    if (nb_local == n / 32 - 1) {
      for (int64_t nb = n / 32; nb < ktiles_col * 8; ++nb)
        s_col[scale_tile_base(band, nb / 8, ktiles_col) + scale_in_tile((int)(kk & 31), (int)(nb & 7))] = 0x7f;
    }
  }
}

}  // namespace mx

// ---------------------------------------------------------------------------------
// Launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------------
hipError_t mx_launch_dim0(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* q, uint8_t* scale,
                          hipStream_t stream) {
  const int64_t row_bands = (rows + 31) / 32, ktiles = mx::scale_tiles_k(cols / 32);
  const int64_t tiles = row_bands * ktiles;
  if (tiles == 0) return hipSuccess;
  const int64_t blocks = (tiles + 3) / 4;
  hipLaunchKernelGGL(mx::k_quant_dim0, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ld, q, scale,
                     row_bands, ktiles);
  return hipGetLastError();
}

hipError_t mx_launch_dim1(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld, uint8_t* q_t,
                          uint8_t* scale_t, hipStream_t stream) {
  const int64_t rtiles = (rows + 255) / 256, ctiles = (cols + 127) / 128;
  const int64_t blocks = batch * rtiles * ctiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx::k_quant_dim1, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ld, q_t,
                     scale_t, rtiles, ctiles);
  return hipGetLastError();
}

hipError_t mx_launch_w32(const uint16_t* w, int64_t batch, int64_t n, int64_t k, int64_t ld, uint8_t* q,
                         uint8_t* q_t, uint8_t* s_row, uint8_t* s_col, hipStream_t stream) {
  const int64_t ktiles = mx::scale_tiles_k(k / 32);
  const int64_t tiles = batch * n / 32 * ktiles;
  if (tiles == 0) return hipSuccess;
  const int64_t blocks = (tiles + 3) / 4;
  hipLaunchKernelGGL(mx::k_quant_w32, dim3((unsigned)blocks), dim3(256), 0, stream, w, batch, n, k, ld, q, q_t,
                     s_row, s_col, ktiles);
  return hipGetLastError();
}
