// MXFP8 training casts for gfx950: dim0 (rowwise 1x32), dim1 (columnwise 32x1,
// written transposed) and the 32x32 weight form.
//
// Numerics (OCP MX): block amax of |x| taken as an unsigned max over the bf16 bit
// patterns with the sign cleared (monotone for finite values); RCEIL E8M0 byte from
// the amax bits by an integer closed form (no division, no log, so no fp32
// flush-to-zero hazard); elements encoded by the gfx950 scaled convert
// (v_cvt_scalef32_pk_fp8_bf16), which computes the RNE E4M3 code of x / 2^(byte-127)
// directly from bf16, two elements per instruction. The convert does not saturate:
// under RCEIL no quotient exceeds 448; under FLOOR the block maximum scales into
// [256, 512) and codes that overflowed to NaN are clamped to +-448 afterwards. Scales are
// written in the MFMA-blocked layout the grouped GEMM reads, so no rearrange pass
// follows (torchtitan PR 5334, body: blocked E8M0 scales emitted directly).
// The bf16 input is read once, with non-temporal loads (keeping it out of the caches
// sped the one-pass cast of the weights from 111 to 103 us inside the MoE step); the
// codes are stored normally, as a GEMM reads them next, except the one-pass cast's
// transposed codes on request (stream_t): those a caller reads only much later are
// stored non-temporally, so the row-wise codes stay cached.

#include <algorithm>
#include <type_traits>

#include "group_table.h"

namespace mx {

// Encode 8 bf16 values (one 16-byte chunk) with scale byte `byte` of a block whose
// amax bits are `amax`: returns 8 codes in two dwords (saturated when SAT).
template <bool SAT>
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
  if (SAT) {
    out.x = sat_e4m3x4(out.x);
    out.y = sat_e4m3x4(out.y);
  }
  return out;
}

// The same for a block whose scale byte is at least 1 (or whose values are all
// zero), given the scale operand: no doubling path.
template <bool SAT>
__device__ inline u32x2 encode8_plain(u32x4 v, float sc) {
  u32x2 out;
  out.x = cvt2(v.x, sc) | (cvt2(v.y, sc) << 16);
  out.y = cvt2(v.z, sc) | (cvt2(v.w, sc) << 16);
  if (SAT) {
    out.x = sat_e4m3x4(out.x);
    out.y = sat_e4m3x4(out.y);
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
// dim0: a wave quantizes 32-row x 256-column tiles (each exactly one 256-byte scale
// tile), striding over the tiles so every wave stays busy to the end and the waves
// of a compute unit drift apart, keeping reads and writes in flight together.
// Lane l reads 16-byte chunk (l % 32) of rows 2i + l/32, i = 0..15; the four lanes
// of a quad hold one 32-element block, reduced with two DPP quad permutes. The
// scale tile is assembled in the wave's own LDS slice (one wave's LDS accesses
// execute in order, so no barrier is needed).
// ---------------------------------------------------------------------------------
template <bool FLOOR>
__global__ __launch_bounds__(256) void k_quant_dim0(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ld, uint8_t* __restrict__ q, uint8_t* __restrict__ scale,
                                                    int64_t row_bands, int64_t ktiles) {
  __shared__ unsigned s_tile[4][64];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, c = l & 31;
  const int64_t tiles = row_bands * ktiles, nwaves = (int64_t)gridDim.x * 4;
  uint8_t* st = (uint8_t*)s_tile[w];
  for (int64_t t = (int64_t)blockIdx.x * 4 + w; t < tiles; t += nwaves) {
    const int64_t rb = t / ktiles, kt = t % ktiles;
    const int64_t col0 = kt * 256 + c * 8;
    const bool col_ok = col0 < cols;
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t r = rb * 32 + 2 * i + h;
      v[i] = (u32x4){0, 0, 0, 0};
      if (col_ok && r < rows) v[i] = __builtin_nontemporal_load((const u32x4*)(x + r * ld + col0));
    }
    s_tile[w][l] = 0x7f7f7f7fu;  // pad bytes of blocks past the last column
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t r = rb * 32 + 2 * i + h;
      unsigned a = amax8(v[i]);
      a = umax(a, dpp_xor1(a));
      a = umax(a, dpp_xor2(a));
      const int byte = scale_byte<FLOOR>(a);
      const u32x2 codes = encode8<FLOOR>(v[i], byte, a);
      if (col_ok && r < rows) {
        *(u32x2*)(q + r * cols + col0) = codes;
        if ((c & 3) == 0) st[scale_in_tile(2 * i + h, c >> 2)] = (uint8_t)byte;
      }
    }
    ((unsigned*)(scale + scale_tile_base(rb, kt, ktiles)))[l] = s_tile[w][l];
  }
}

// ---------------------------------------------------------------------------------
// dim1: a workgroup quantizes a 256-row x 64-column tile of one batch: eight 32-row
// blocks of each of 64 columns, which become 64 rows of q_t with 256 contiguous
// codes each, and two full 256-byte scale tiles.
//   Loads: lane l takes columns 8(l%8)..+7 (16 bytes); wave w, block half hb and
//   i = 0..3 give row 64w + 32hb + 4(l/8) + i, so one load instruction reads eight
//   rows x 128 bytes (whole lines) and a lane holds 4 consecutive rows of each of
//   its two blocks.
//   Amax: per column over the lane's 4 rows, then across the 8 lanes of its column
//   group (lane bits 3..5).
//   Encode: the same column of two rows forms one converter pair, so each column's
//   4 rows come out as one dword of the transposed tile.
//   Transpose: the 64 x 256-byte code tile sits in LDS with row c's bytes r XOR-ed
//   by ((c / 8) % 8) * 32, so the dword writes (64 lanes, 64 banks) and the 16-byte
//   row reads are both conflict-free; the stores then write 256-byte rows of q_t.
// ---------------------------------------------------------------------------------
template <bool FLOOR>
__global__ __launch_bounds__(256) void k_quant_dim1(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ld, uint8_t* __restrict__ q_t,
                                                    uint8_t* __restrict__ scale_t, int64_t rtiles, int64_t ctiles) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[64 * 256];
  __shared__ unsigned s_scale[2][64];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, cg = l & 7, g = l >> 3;
  const int64_t bid = blockIdx.x;
  const int64_t b = bid / (rtiles * ctiles);
  const int64_t rem = bid % (rtiles * ctiles);
  const int64_t ct = rem / rtiles, rt = rem % rtiles;
  const int64_t r0 = rt * 256, c0 = ct * 64;
  const int64_t cl = c0 + 8 * cg;
  const bool col_ok = cl < cols;  // cols % 32 == 0: a lane's 8 columns are all in or all out
  const uint16_t* xb = x + b * rows * ld;
  if (tid < 128) s_scale[tid >> 6][tid & 63] = 0x7f7f7f7fu;  // pad blocks past the last row

  u32x4 v[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + 64 * w + 32 * hb + 4 * g + i;
      v[hb][i] = (u32x4){0, 0, 0, 0};
      if (col_ok && r < rows) v[hb][i] = __builtin_nontemporal_load((const u32x4*)(xb + r * ld + cl));
    }
  __syncthreads();  // pad fill of the scale tiles before the byte writes

  uint8_t* ssc = (uint8_t*)s_scale;
  const int swz = cg << 5;  // XOR applied to the row byte of code-tile rows 8cg..8cg+7
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int kb = 2 * w + hb;              // block within the tile (input rows 32kb..32kb+31)
    const int rloc = 64 * w + 32 * hb + 4 * g;  // the lane's first row within the tile
    // packed amax of column pairs (2p, 2p+1), p = 0..3
    unsigned am[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      unsigned a = amax_pair(0u, v[hb][0][p]);
      a = amax_pair(a, v[hb][1][p]);
      a = amax_pair(a, v[hb][2][p]);
      a = amax_pair(a, v[hb][3][p]);
      a = amax_pair(a, (unsigned)__builtin_amdgcn_mov_dpp((int)a, 0x128, 0xF, 0xF, false));  // lane ^ 8
      a = amax_pair(a, (unsigned)__shfl_xor((int)a, 16));
      a = amax_pair(a, (unsigned)__shfl_xor((int)a, 32));
      am[p] = a;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {  // column 2p + e of the lane's eight
        const unsigned amax = e ? (am[p] >> 16) : (am[p] & 0xffff);
        const int byte = scale_byte<FLOOR>(amax);
        const bool tiny = byte == 0 && amax != 0;
        const float sc = scale_operand(byte == 0 ? 1 : byte);
        const unsigned sel = e ? 0x07060302u : 0x05040100u;
        unsigned p01 = __builtin_amdgcn_perm(v[hb][1][p], v[hb][0][p], sel);  // (row 0, row 1) of the column
        unsigned p23 = __builtin_amdgcn_perm(v[hb][3][p], v[hb][2][p], sel);
        if (tiny) {
          p01 = double_bf16x2(p01);
          p23 = double_bf16x2(p23);
        }
        unsigned codes = cvt2(p01, sc) | (cvt2(p23, sc) << 16);
        if (FLOOR) codes = sat_e4m3x4(codes);
        const int c = 8 * cg + 2 * p + e;  // column within the tile = row of the code tile
        *(unsigned*)(s_codes + c * 256 + (rloc ^ swz)) = codes;
        if (g == 0 && r0 + 32 * kb < rows) ssc[(c >> 5) * 256 + scale_in_tile(c & 31, kb)] = (uint8_t)byte;
      }
    }
  }
  __syncthreads();

  // q_t rows c0 + 16w .. +15, four per instruction, 16 lanes x 16 bytes each
  uint8_t* qb = q_t + b * cols * rows;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int orow = 16 * w + 4 * k + (l >> 4), chunk = l & 15;
    const int64_t c = c0 + orow, rr = r0 + 16 * chunk;
    const u32x4 d = *(const u32x4*)(s_codes + orow * 256 + ((chunk ^ (((orow >> 3) & 7) << 1)) << 4));
    if (c < cols && rr < rows) *(u32x4*)(qb + c * rows + rr) = d;
  }
  if (tid < 128) {
    const int tile = tid >> 6;
    const int64_t out_row0 = c0 + 32 * tile;  // first q_t row of this scale tile
    if (out_row0 < cols) {
      const int64_t band = (b * cols + out_row0) / 32;
      const int64_t ktiles = scale_tiles_k(rows / 32);
      ((unsigned*)(scale_t + scale_tile_base(band, rt, ktiles)))[tid & 63] = s_scale[tile][tid & 63];
    }
  }
}

// ---------------------------------------------------------------------------------
// dim0 + dim1 in one pass: a workgroup reads a 256-row x 256-column tile of one batch
// once and writes both casts (4.0625 B per element instead of 2 x 3.03125).
//   With four waves, wave w takes rows 64w..64w+63 as two 32-row sub-tiles in turn;
//   with eight, wave w takes rows 32w..32w+31. In a sub-tile lane l
//   reads 16-byte chunk (l % 32) of rows 16(l/32) + i, i = 0..15 (two rows x 512
//   bytes per load instruction).
//   dim0: as k_quant_dim0 (quad amax per row block, codes to q, the sub-tile's
//   256-byte scale tile assembled in the wave's LDS slice).
//   dim1: per column, amax over the lane's 16 rows then with lane l ^ 32; adjacent
//   rows of one column form each converter pair, so a column's 16 codes are 16
//   contiguous bytes of its q_t row; they go to a 256 x 256-byte LDS tile (row =
//   column of the tile, 16-byte chunk k at k ^ ((row / 8) % 16): conflict-free), read
//   back as whole 256-byte q_t rows. The eight dim1 scale tiles (256 columns x 8
//   blocks) are assembled in LDS and written whole.
// GATHER (token-group padding fused in, one 2D input): `rows` counts the padded rows;
// padded row p holds row padded_source(p) of x, or zeros (ao fork PR 10, "Known
// follow-ups": padded token groups), so the padded bf16 copy is never written.
// ---------------------------------------------------------------------------------
// A raw buffer from `base` for the one-pass cast's loads and stores: lanes outside
// the tensor take the offset kOutside, which the range check drops (stores) or reads
// as zeros (loads), so no lane needs a branch; the row-dependent part of an address
// goes in the scalar offset, so a lane holds one 32-bit offset for all 16 rows
// (64-bit addresses for 16 loads and 16 stores took 64 VGPRs). Every in-range offset
// is below 2^31 for row strides up to 2^25 elements (checked on the host).
constexpr uint32_t kOutside = 0x80000000u;
__device__ inline __amdgpu_buffer_rsrc_t cast_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, 0x00020000);
}

struct RowGather {
  const int32_t* offs;  // unpadded group ends (device)
  int groups;
  int32_t src_rows;     // rows of x
  int32_t* offs_pad;    // padded group ends (written by workgroup 0)
};

template <bool FLOOR, bool GATHER, int WV>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(2))) void k_quant_both(const uint16_t* __restrict__ x, int64_t batch, int64_t rows,
                                                    int64_t cols, int64_t ld, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ scale, uint8_t* __restrict__ q_t,
                                                    uint8_t* __restrict__ scale_t, int64_t rtiles, int64_t ctiles,
                                                    RowGather gth, int stream_t) {
  __shared__ __attribute__((aligned(16))) uint8_t s_t[256 * 256];  // transposed codes
  __shared__ unsigned s_s1[8][64];                                 // dim1 scale tiles
  __shared__ unsigned s_s0[WV][64];                                // dim0 scale tile per wave
  constexpr int SUBS = 8 / WV;  // 32-row sub-tiles per wave, one after the other
  __shared__ std::conditional_t<GATHER, GroupTable, char> s_grp;  // the group table (gather only)
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, c = l & 31;
  if constexpr (GATHER) {
    build_table(s_grp, gth.offs, gth.groups, gth.src_rows);
    if (blockIdx.x == 0)
      for (int g = tid; g < gth.groups; g += 64 * WV) gth.offs_pad[g] = s_grp.pad_end[g];
  }
  const int64_t kt0 = scale_tiles_k(cols / 32), kt1 = scale_tiles_k(rows / 32);
  const int64_t tiles = batch * rtiles * ctiles;
  uint8_t* st0 = (uint8_t*)s_s0[w];
  uint8_t* ss1 = (uint8_t*)s_s1;

  // The wave's sub-tile `sub` of tile t: its 16 loads (zeros outside the tensor or
  // past the last tile).
  auto load = [&](u32x4(&v)[16], int64_t t, int sub) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (u32x4){0, 0, 0, 0};
    if (t >= tiles) return;
    const int64_t b = t / (rtiles * ctiles), rem = t % (rtiles * ctiles);
    const int64_t r0 = (rem % rtiles) * 256, col = (rem / rtiles) * 256 + 8 * c;
    const int64_t base = r0 + 32 * (SUBS * w + sub);
    if (base >= rows) return;  // rows % 32 == 0: the sub-tile is all in or all out
    const uint32_t lane_off = col < cols ? (uint32_t)((16 * h * ld + col) * 2) : kOutside;
    if constexpr (GATHER) {
      // The sub-tile's 32 rows form one 32-row block of the padded rows, and padded
      // group edges are multiples of 32, so they lie in one padded group: a single
      // lookup gives the run of source rows, read as one run (a pointer per load needed
      // 301 VGPRs, one workgroup per compute unit, 94 us; walking group edges row by
      // row between loads, 78 us; one lookup, 69 us, on the MoE tokens, same device).
      const GroupTable& gt = s_grp;
      const int g = upper_index(gt.pad_end, gth.groups, base);
      int64_t src0 = 0, real = 0;  // source row of padded row `base`; real rows from it on
      if (g < gth.groups) {
        src0 = (g ? gt.end[g - 1] : 0) + (base - (g ? gt.pad_end[g - 1] : 0));
        real = gt.end[g] - src0;
      }
      if (real <= 0) src0 = 0;
      src0 = __builtin_amdgcn_readfirstlane((int)src0);  // the same in every lane
      const int nreal = real <= 16 * h ? 0 : (real - 16 * h < 16 ? (int)(real - 16 * h) : 16);  // the lane's real rows
      const auto rx = cast_rsrc(x + src0 * ld);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, i < nreal ? lane_off : kOutside, (int)(i * ld * 2), 2);
    } else {
      const auto rx = cast_rsrc(x + (b * rows + base) * ld);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, lane_off, (int)(i * ld * 2), 2);
    }
  };

  // Each wave keeps its next sub-tile's loads in flight while it encodes the current
  // one, and the first sub-tile of its next tile in flight across the barrier and the
  // q_t stores that end a tile, so the bf16 reads never wait on the encode or the
  // stores.
  u32x4 v[16];
  load(v, blockIdx.x, 0);
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t b = t / (rtiles * ctiles), rem = t % (rtiles * ctiles);
    const int64_t ct = rem / rtiles, rt = rem % rtiles;
    const int64_t r0 = rt * 256, c0 = ct * 256;
    const int64_t col = c0 + 8 * c;
    const bool col_ok = col < cols;  // cols % 32 == 0: a quad's 32 columns are all in or all out
    const int64_t qrow0 = b * rows;  // dim0 rows of this batch in the stacked [batch*rows x cols]
    for (int i = tid; i < 8 * 64; i += 64 * WV) s_s1[i >> 6][i & 63] = 0x7f7f7f7fu;  // pad blocks past the last row
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < SUBS; ++sub) {
      const int kb = SUBS * w + sub;            // dim1 block (32 rows) within the tile
      const int64_t base = r0 + 32 * kb;        // first row of the sub-tile
      const bool rows_ok = base < rows;         // rows % 32 == 0: the sub-tile is all in or all out
      u32x4 nv[16];
      if (sub + 1 < SUBS)
        load(nv, t, sub + 1);
      else
        load(nv, t + gridDim.x, 0);
      // the block amaxes of both casts from one pass over |v|: each row's 8 values
      // (dim0, reduced over the quad below) and the lane's column pairs over its 16
      // rows (dim1), so no |v| stays live between the two casts
      unsigned a0[16], am[4] = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        unsigned r = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          r = amax_pair(r, v[i][p]);
          am[p] = amax_pair(am[p], v[i][p]);
        }
        a0[i] = fold_pair(r);
      }
      // ---- dim0 ----
      s_s0[w][l] = 0x7f7f7f7fu;
      const auto rq = cast_rsrc(q + (qrow0 + base) * cols);
      const uint32_t q_off = col_ok ? (uint32_t)(16 * h * cols + col) : kOutside;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        unsigned a = a0[i];
        a = umax(a, dpp_xor1(a));
        a = umax(a, dpp_xor2(a));
        const int byte = scale_byte<FLOOR>(a);
        // a scale byte of 0 with a non-zero amax (tiny values) needs the doubling
        // path; a wave that has none takes the short one
        u32x2 codes;
        if (__builtin_expect(__ballot(byte == 0 && a != 0) == 0, 1))
          codes = encode8_plain<FLOOR>(v[i], scale_operand(byte == 0 ? 1 : byte));
        else
          codes = encode8<FLOOR>(v[i], byte, a);
        if (rows_ok) {
          __builtin_amdgcn_raw_buffer_store_b64(codes, rq, q_off, (int)(i * cols), 0);
          if (col_ok && (c & 3) == 0) st0[scale_in_tile(16 * h + i, c >> 2)] = (uint8_t)byte;
        }
      }
      if (rows_ok && c0 < cols)
        __builtin_amdgcn_raw_buffer_store_b32(s_s0[w][l], cast_rsrc(scale + scale_tile_base((qrow0 + base) / 32, ct, kt0)),
                                              4 * l, 0, 0);
      // ---- dim1 ----
#pragma unroll
      for (int p = 0; p < 4; ++p) {  // column pair (2p, 2p+1) of the lane's eight
        const unsigned a32 = amax_pair(am[p], (unsigned)__shfl_xor((int)am[p], 32));
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const unsigned amax = e ? (a32 >> 16) : (a32 & 0xffff);
          const int byte = scale_byte<FLOOR>(amax);
          const bool tiny = byte == 0 && amax != 0;
          const float sc = scale_operand(byte == 0 ? 1 : byte);
          const unsigned sel = e ? 0x07060302u : 0x05040100u;
          unsigned d[4];
          if (__builtin_expect(__ballot(tiny) == 0, 1)) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const unsigned p01 = __builtin_amdgcn_perm(v[4 * m + 1][p], v[4 * m][p], sel);  // rows 4m, 4m+1
              const unsigned p23 = __builtin_amdgcn_perm(v[4 * m + 3][p], v[4 * m + 2][p], sel);
              d[m] = cvt2(p01, sc) | (cvt2(p23, sc) << 16);
            }
          } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              unsigned p01 = __builtin_amdgcn_perm(v[4 * m + 1][p], v[4 * m][p], sel);
              unsigned p23 = __builtin_amdgcn_perm(v[4 * m + 3][p], v[4 * m + 2][p], sel);
              if (tiny) {
                p01 = double_bf16x2(p01);
                p23 = double_bf16x2(p23);
              }
              d[m] = cvt2(p01, sc) | (cvt2(p23, sc) << 16);
            }
          }
          if (FLOOR) {
#pragma unroll
            for (int m = 0; m < 4; ++m) d[m] = sat_e4m3x4(d[m]);
          }
          const int cc = 8 * c + 2 * p + e;      // column within the tile = row of s_t
          const int k = 2 * kb + h;  // 16-byte chunk: the lane's 16 rows
          *(u32x4*)(s_t + cc * 256 + ((k ^ ((cc >> 3) & 15)) << 4)) = (u32x4){d[0], d[1], d[2], d[3]};
          if (h == 0 && rows_ok) ss1[(cc >> 5) * 256 + scale_in_tile(cc & 31, kb)] = (uint8_t)byte;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = nv[i];
    }
    __syncthreads();
    // q_t rows c0 + (256/WV)w .. (columns of the tile), four per instruction, 256 bytes
    // each: row c0 + orow0 + (l >> 4) from a per-instruction base, so a lane's offset
    // stays below 4 * rows + 256
    {
      const int ch = l & 15;
      const uint32_t lane_off = r0 + 16 * ch < rows ? (uint32_t)((l >> 4) * rows + 16 * ch) : kOutside;
#pragma unroll
      for (int k = 0; k < 64 / WV; ++k) {
        const int orow0 = 256 / WV * w + 4 * k, orow = orow0 + (l >> 4);
        const u32x4 d = *(const u32x4*)(s_t + orow * 256 + ((ch ^ ((orow >> 3) & 15)) << 4));
        if (c0 + orow0 < cols) {  // cols % 32 == 0: the four rows are all in or all out
          const auto rqt = cast_rsrc(q_t + (b * cols + c0 + orow0) * rows + r0);
          if (stream_t)
            __builtin_amdgcn_raw_buffer_store_b128(d, rqt, lane_off, 0, 2);  // non-temporal
          else
            __builtin_amdgcn_raw_buffer_store_b128(d, rqt, lane_off, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8 / WV; ++j) {
      const int tile = WV * j + w;  // dim1 scale tile (32 q_t rows) of this thread's dword
      const int64_t out_row0 = c0 + 32 * tile;
      if (out_row0 < cols)
        __builtin_amdgcn_raw_buffer_store_b32(s_s1[tile][l], cast_rsrc(scale_t + scale_tile_base((b * cols + out_row0) / 32, rt, kt1)),
                                              4 * l, 0, 0);
    }
    __syncthreads();  // s_t and s_s1 are reused by the next tile
  }
}

// ---------------------------------------------------------------------------------
// 32x32 weight cast: one wave per 32-row x 64-column strip (two 32x32 tiles), four
// independent waves per workgroup, so a narrow weight still spreads over every
// compute unit (the 576 x 4096 weight: 1152 strips). Lane l holds 16-byte column
// chunk l % 8 of rows l / 8 + 8i, i = 0..3. The tile amax reduces over the lane's 4
// rows, the quad (the tile's 32 columns) and the 8 row groups. Codes go out rowwise
// directly and, through the wave's LDS slice, transposed: each lane turns 8 rows x 4
// columns into 8 bytes of 4 q_t rows with byte permutes.
// ---------------------------------------------------------------------------------
constexpr int kW32Waves = 4;  // waves per workgroup (independent strips)

__global__ __launch_bounds__(64 * kW32Waves) void k_quant_w32(const uint16_t* __restrict__ w, int64_t batch, int64_t n,
                                                   int64_t k, int64_t ld, uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ q_t, uint8_t* __restrict__ s_row,
                                                   uint8_t* __restrict__ s_col, int64_t ktiles) {
  __shared__ unsigned lds_q[kW32Waves][32 * 16];  // per wave: 32 rows x 64 bytes of codes
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 7, g = l >> 3;
  const int64_t strips_k = (k + 63) / 64, row_bands = batch * n / 32;
  const int64_t t = (int64_t)blockIdx.x * kW32Waves + wv;
  const bool active = t < row_bands * strips_k;
  const int64_t rb = active ? t / strips_k : 0, col0 = active ? (t % strips_k) * 64 : 0;
  const int64_t col = col0 + 8 * c;
  const bool col_ok = active && col < k;  // k % 32 == 0: a tile is all in or all out
  const int kb_total = (int)(k / 32);

  u32x4 v[4];
  unsigned a = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (u32x4){0, 0, 0, 0};
    if (col_ok) v[i] = __builtin_nontemporal_load((const u32x4*)(w + (rb * 32 + g + 8 * i) * ld + col));
    a = umax(a, amax8(v[i]));
  }
  a = umax(a, dpp_xor1(a));
  a = umax(a, dpp_xor2(a));
  a = umax(a, (unsigned)__shfl_xor((int)a, 8));
  a = umax(a, (unsigned)__shfl_xor((int)a, 16));
  a = umax(a, (unsigned)__shfl_xor((int)a, 32));
  const int byte = rceil_byte(a);
  const int tb0 = __shfl(byte, 0), tb1 = __shfl(byte, 4);  // the strip's two tile bytes

  uint8_t* lq = (uint8_t*)lds_q[wv];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x2 codes = encode8<false>(v[i], byte, a);
    if (col_ok) *(u32x2*)(q + (rb * 32 + g + 8 * i) * k + col) = codes;
    *(u32x2*)(lq + (g + 8 * i) * 64 + c * 8) = codes;
  }
  __syncthreads();
  if (!active) return;
  // rowwise scales: row l % 32 of the band, block col0/32 + l/32; the strip that ends
  // the row also fills the layout's pad blocks up to a multiple of eight
  {
    const int kb = (int)(col0 / 32) + (l >> 5);
    if (kb < kb_total) s_row[scale_tile_base(rb, kb / 8, ktiles) + scale_in_tile(l & 31, kb & 7)] = (uint8_t)((l >> 5) ? tb1 : tb0);
    if (col0 + 64 >= k)
      for (int kp = kb_total + (l >> 5); kp < ktiles * 8; kp += 2)
        s_row[scale_tile_base(rb, kp / 8, ktiles) + scale_in_tile(l & 31, kp & 7)] = 0x7f;
  }
  if (q_t == nullptr) return;
  // transposed codes: lane l takes columns 4 (l % 16) .. +3 of rows 8 (l / 16) .. +7
  // and writes 8 bytes of each of those 4 q_t rows
  const int dc = l & 15, p8 = l >> 4;
  unsigned outw[2][4];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r0 = 8 * p8 + 4 * half;
    const unsigned d0 = lds_q[wv][(r0 + 0) * 16 + dc];
    const unsigned d1 = lds_q[wv][(r0 + 1) * 16 + dc];
    const unsigned d2 = lds_q[wv][(r0 + 2) * 16 + dc];
    const unsigned d3 = lds_q[wv][(r0 + 3) * 16 + dc];
    const unsigned t0 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
    const unsigned t1 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
    const unsigned t2 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
    const unsigned t3 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
    outw[half][0] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
    outw[half][1] = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
    outw[half][2] = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
    outw[half][3] = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
  }
  const int64_t bi = (rb * 32) / n;
  const int64_t nb_local = (rb * 32 - bi * n) / 32;  // 32-column band of q_t within the batch
  uint8_t* qtb = q_t + bi * k * n;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t kk = col0 + 4 * dc + j;
    if (kk < k) *(u32x2*)(qtb + kk * n + nb_local * 32 + 8 * p8) = (u32x2){outw[0][j], outw[1][j]};
  }
  // column scales: q_t row col0 + l, block nb_local (the band's 32 columns); the last
  // band of the batch also fills the layout's pad blocks
  const int64_t kk = col0 + l;
  if (kk < k) {
    const int64_t ktiles_col = scale_tiles_k(n / 32);
    const int64_t band = (bi * k + kk) / 32;
    s_col[scale_tile_base(band, nb_local / 8, ktiles_col) + scale_in_tile((int)(kk & 31), (int)(nb_local & 7))] =
        (uint8_t)((l >> 5) ? tb1 : tb0);
    if (nb_local == n / 32 - 1)
      for (int64_t nb = n / 32; nb < ktiles_col * 8; ++nb)
        s_col[scale_tile_base(band, nb / 8, ktiles_col) + scale_in_tile((int)(kk & 31), (int)(nb & 7))] = 0x7f;
  }
}

}  // namespace mx

// ---------------------------------------------------------------------------------
// Launchers (called by the C ABI after validation)
// ---------------------------------------------------------------------------------

namespace {
// Blocks that fill the current device once: resident blocks per compute unit for
// this kernel (from its register and LDS use) times the compute units.
int64_t resident_blocks(const void* kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0) per_cu = 1;
  return (int64_t)cus * per_cu;
}
}  // namespace
hipError_t mx_launch_dim0(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* q, uint8_t* scale,
                          int floor_mode, hipStream_t stream) {
  const int64_t row_bands = (rows + 31) / 32, ktiles = mx::scale_tiles_k(cols / 32);
  const int64_t tiles = row_bands * ktiles;
  if (tiles == 0) return hipSuccess;
  // enough 4-wave blocks to fill the device once, each wave striding over the tiles
  // per process (thread-safe static initialisation); every gfx950 part has the same shape
  static const int64_t fill = resident_blocks((const void*)mx::k_quant_dim0<false>, 256);
  const int64_t blocks = std::min<int64_t>((tiles + 3) / 4, fill);
  if (floor_mode)
    hipLaunchKernelGGL(mx::k_quant_dim0<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ld, q,
                       scale, row_bands, ktiles);
  else
    hipLaunchKernelGGL(mx::k_quant_dim0<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ld, q,
                       scale, row_bands, ktiles);
  return hipGetLastError();
}

hipError_t mx_launch_dim1(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld, uint8_t* q_t,
                          uint8_t* scale_t, int floor_mode, hipStream_t stream) {
  const int64_t rtiles = (rows + 255) / 256, ctiles = (cols + 63) / 64;
  const int64_t blocks = batch * rtiles * ctiles;
  if (blocks == 0) return hipSuccess;
  if (floor_mode)
    hipLaunchKernelGGL(mx::k_quant_dim1<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ld, q_t,
                       scale_t, rtiles, ctiles);
  else
    hipLaunchKernelGGL(mx::k_quant_dim1<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, cols, ld, q_t,
                       scale_t, rtiles, ctiles);
  return hipGetLastError();
}

namespace {
// One launch of the one-pass cast with WV waves per workgroup: at most one
// workgroup per resident slot, each walking tiles.
template <bool FLOOR, bool GATHER, int WV>
hipError_t launch_both_wv(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld, uint8_t* q,
                          uint8_t* scale, uint8_t* q_t, uint8_t* scale_t, int64_t rtiles, int64_t ctiles,
                          mx::RowGather gth, int stream_t, hipStream_t stream) {
  static const int64_t fill = resident_blocks((const void*)mx::k_quant_both<FLOOR, GATHER, WV>, 64 * WV);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(batch * rtiles * ctiles, fill));
  hipLaunchKernelGGL((mx::k_quant_both<FLOOR, GATHER, WV>), dim3((unsigned)blocks), dim3(64 * WV), 0, stream, x,
                     batch, rows, cols, ld, q, scale, q_t, scale_t, rtiles, ctiles, gth, stream_t);
  return hipGetLastError();
}

// Waves per workgroup of the one-pass cast for `tiles` 256x256 tiles. Four waves
// (each two 32-row sub-tiles in turn), two workgroups per compute unit, whose
// phases overlap; where there is at most one tile per compute unit, eight waves
// (one sub-tile each) finish a tile sooner (16384 x 576 grad_out: 14 against 18 us;
// 16384 x 4096: 70 against 58 us).
int both_waves(int64_t tiles) {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    return n;
  }();
  return tiles <= cus ? 8 : 4;
}
}  // namespace

hipError_t mx_launch_both(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld, uint8_t* q,
                          uint8_t* scale, uint8_t* q_t, uint8_t* scale_t, int floor_mode, int stream_t,
                          hipStream_t stream) {
  const int64_t rtiles = (rows + 255) / 256, ctiles = (cols + 255) / 256;
  const int64_t tiles = batch * rtiles * ctiles;
  if (tiles == 0) return hipSuccess;
  const mx::RowGather none{nullptr, 0, 0, nullptr};
  const bool eight = both_waves(tiles) == 8;
  if (floor_mode)
    return eight ? launch_both_wv<true, false, 8>(x, batch, rows, cols, ld, q, scale, q_t, scale_t, rtiles, ctiles, none, stream_t, stream)
                 : launch_both_wv<true, false, 4>(x, batch, rows, cols, ld, q, scale, q_t, scale_t, rtiles, ctiles, none, stream_t, stream);
  return eight ? launch_both_wv<false, false, 8>(x, batch, rows, cols, ld, q, scale, q_t, scale_t, rtiles, ctiles, none, stream_t, stream)
               : launch_both_wv<false, false, 4>(x, batch, rows, cols, ld, q, scale, q_t, scale_t, rtiles, ctiles, none, stream_t, stream);
}

// Padded one-pass cast: x [rows x cols] with unpadded group ends offs -> codes of the
// [rows_pad x cols] padded rows (both forms), offs_pad written (one workgroup is
// launched even for no tiles, to write offs_pad).
hipError_t mx_launch_pad_both(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const int32_t* offs,
                              int groups, int64_t rows_pad, uint8_t* q, uint8_t* scale, uint8_t* q_t,
                              uint8_t* scale_t, int32_t* offs_pad, int stream_t, hipStream_t stream) {
  const int64_t rtiles = (rows_pad + 255) / 256, ctiles = (cols + 255) / 256;
  const mx::RowGather gth{offs, groups, (int32_t)rows, offs_pad};
  if (both_waves(rtiles * ctiles) == 8)
    return launch_both_wv<false, true, 8>(x, 1, rows_pad, cols, ld, q, scale, q_t, scale_t, rtiles, ctiles, gth, stream_t, stream);
  return launch_both_wv<false, true, 4>(x, 1, rows_pad, cols, ld, q, scale, q_t, scale_t, rtiles, ctiles, gth, stream_t, stream);
}

hipError_t mx_launch_w32(const uint16_t* w, int64_t batch, int64_t n, int64_t k, int64_t ld, uint8_t* q,
                         uint8_t* q_t, uint8_t* s_row, uint8_t* s_col, hipStream_t stream) {
  const int64_t ktiles = mx::scale_tiles_k(k / 32);
  const int64_t strips = batch * n / 32 * ((k + 63) / 64);
  if (strips == 0) return hipSuccess;
  const int64_t blocks = (strips + mx::kW32Waves - 1) / mx::kW32Waves;
  hipLaunchKernelGGL(mx::k_quant_w32, dim3((unsigned)blocks), dim3(64 * mx::kW32Waves), 0, stream, w, batch, n, k, ld,
                     q, q_t,
                     s_row, s_col, ktiles);
  return hipGetLastError();
}
