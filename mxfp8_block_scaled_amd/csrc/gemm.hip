// MXFP8 scaled grouped GEMM for gfx950 on the block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, E8M0 scale per 32-block, fp32
// accumulation).
//
// One core computes C[i, j] = sum_c A[i, c] * B[j, c] with both operands stored
// contraction-contiguous; the three passes differ only in how tiles map to groups:
//   M-grouped (forward, dgrad): group g owns rows [offs[g-1], offs[g]) of A and
//     the [N x K] slab g of B; every group contracts over all of K.
//   K-grouped (wgrad): every group sees all rows of A and B but contracts over
//     its own range [offs[g-1], offs[g]) of the shared contraction axis; an empty
//     range leaves zeros.
// The grouped GEMM with offs per expert is the MoE form; offs = NULL is the dense
// layer (torchtitan PR 5334, body: one API for dense and grouped).
//
// MFMA operand layout (measured on gfx950): lane l holds row l % 32 of a 32-row
// operand tile; its 32 bytes are the contraction elements [16h, 16h+16) and
// [32+16h, 32+16h+16) of the 64-wide k-step, h = l / 32. The scale of row r and
// k-block b (0/1) of the step comes from lane r + 32b, byte `opsel`. The output
// 32x32 tile: lane l, register v -> row 8*(v/4) + 4*h + v%4, column l % 32.

#include "common.h"

namespace mx {

enum { MODE_MGROUP = 0, MODE_KGROUP = 1 };

struct GemmArgs {
  const uint8_t* a;    // [a_rows x lda] codes
  const uint8_t* a_s;  // MFMA-blocked scales of a
  const uint8_t* b;
  const uint8_t* b_s;
  const int32_t* offs;  // device, may be null (one group)
  void* out;
  int64_t lda, ldb;          // row pitch in bytes (= contraction length)
  int64_t a_rows, b_rows;    // rows of the whole operand buffers
  int64_t a_ktiles, b_ktiles;  // scale tiles along the contraction
  int64_t M, N, K;  // M-grouped: M = token rows, N = per-group output columns, K = contraction
                    // K-grouped: M = rows of A, N = rows of B, K = contraction (tokens)
  int64_t ldo;      // output row pitch (elements)
  int64_t mt_total, nt;  // tile grid: m-tiles (upper bound for M-grouped), n-tiles
  int groups;
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
struct Cfg {
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M;  // rows per wave
  static constexpr int WN = BN / WAVES_N;
  static constexpr int TM = WM / 32;  // 32x32 MFMA tiles per wave
  static constexpr int TN = WN / 32;
  static constexpr int KSTEPS = BK / 64;
  static constexpr int CHUNKS_ROW = BK / 16;
  static constexpr int A_CHUNKS = BM * CHUNKS_ROW / THREADS;  // 16-byte chunks per thread
  static constexpr int B_CHUNKS = BN * CHUNKS_ROW / THREADS;
  static constexpr int A_BYTES = BM * BK;
  static constexpr int B_BYTES = BN * BK;
  static_assert(BK == 128, "scale handling assumes two 128-wide k-tiles per 256-wide scale tile");
  static_assert(A_CHUNKS * THREADS == BM * CHUNKS_ROW && B_CHUNKS * THREADS == BN * CHUNKS_ROW, "");
};

// XOR swizzle of the 16-byte chunk within a row (8 chunks per 128-byte row).
__device__ inline int lds_off(int row, int kc) { return row * 128 + ((kc ^ (row & 7)) << 4); }

__device__ inline int32_t group_start(const int32_t* offs, int g) { return g == 0 ? 0 : offs[g - 1]; }

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int MODE, int OUT_BF16>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm(GemmArgs p) {
  using C = Cfg<BM, BN, BK, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][C::A_BYTES + C::B_BYTES];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, h = l >> 5;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---- tile id: spread consecutive tiles over one XCD (blocks are dealt
  // round-robin to the 8 XCDs), then a grouped raster of 8 m-tiles.
  const int64_t nblk = gridDim.x, bid = blockIdx.x;
  const int64_t per_xcd = nblk / 8;
  const int64_t lid = bid < per_xcd * 8 ? (bid % 8) * per_xcd + bid / 8 : bid;

  int g = 0;
  int64_t m_tile, n_tile;
  int64_t a_row0, a_row_end, b_row0, b_row_end, k_beg, k_end, out_row0;
  uint8_t* out_base = (uint8_t*)p.out;
  const int out_es = OUT_BF16 ? 2 : 4;
  if (MODE == MODE_MGROUP) {
    const int64_t GM = 8;
    const int64_t band = lid / (GM * p.nt);
    const int64_t first_m = band * GM;
    const int64_t gm = p.mt_total - first_m < GM ? p.mt_total - first_m : GM;
    const int64_t in_band = lid % (GM * p.nt);
    const int64_t mt_glob = first_m + in_band % gm;
    n_tile = in_band / gm;
    // find the group that owns this m-tile
    int64_t cum = 0;
    int found = -1;
    int64_t local = 0;
    const int G = p.offs ? p.groups : 1;
    for (int gg = 0; gg < G; ++gg) {
      const int64_t s = p.offs ? group_start(p.offs, gg) : 0;
      const int64_t e = p.offs ? p.offs[gg] : p.M;
      const int64_t tiles = (e - s + BM - 1) / BM;
      if (mt_glob < cum + tiles) {
        found = gg;
        local = mt_glob - cum;
        a_row0 = s + local * BM;
        a_row_end = e;
        break;
      }
      cum += tiles;
    }
    if (found < 0) return;
    g = found;
    m_tile = local;
    b_row0 = (int64_t)g * p.N + n_tile * BN;
    b_row_end = (int64_t)g * p.N + p.N;
    k_beg = 0;
    k_end = p.K;
    out_row0 = a_row0;
  } else {
    const int64_t per_g = p.mt_total * p.nt;
    g = (int)(lid / per_g);
    const int64_t r = lid % per_g;
    const int64_t GM = 8;
    const int64_t band = r / (GM * p.nt);
    const int64_t first_m = band * GM;
    const int64_t gm = p.mt_total - first_m < GM ? p.mt_total - first_m : GM;
    const int64_t in_band = r % (GM * p.nt);
    m_tile = first_m + in_band % gm;
    n_tile = in_band / gm;
    a_row0 = m_tile * BM;
    a_row_end = p.M;
    b_row0 = n_tile * BN;
    b_row_end = p.N;
    k_beg = p.offs ? group_start(p.offs, g) : 0;
    k_end = p.offs ? p.offs[g] : p.K;
    out_row0 = a_row0;
    out_base += (int64_t)g * p.M * p.ldo * out_es;
  }
  const int64_t col0 = n_tile * BN;                            // output column of the tile
  const int64_t n_limit = MODE == MODE_MGROUP ? p.N : p.N;     // columns per output row

  // ---- global -> register staging (16-byte chunks) --------------------------------
  u32x4 ra[C::A_CHUNKS], rb[C::B_CHUNKS];
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) {
      const int id = tid + i * C::THREADS;
      const int row = id / C::CHUNKS_ROW, kc = id % C::CHUNKS_ROW;
      const int64_t gr = a_row0 + row, kk = k0 + kc * 16;
      ra[i] = (u32x4){0, 0, 0, 0};
      if (gr < a_row_end && gr < p.a_rows && kk >= k_beg && kk < k_end) ra[i] = *(const u32x4*)(p.a + gr * p.lda + kk);
    }
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) {
      const int id = tid + i * C::THREADS;
      const int row = id / C::CHUNKS_ROW, kc = id % C::CHUNKS_ROW;
      const int64_t gr = b_row0 + row, kk = k0 + kc * 16;
      rb[i] = (u32x4){0, 0, 0, 0};
      if (gr < b_row_end && gr < p.b_rows && kk >= k_beg && kk < k_end) rb[i] = *(const u32x4*)(p.b + gr * p.ldb + kk);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) {
      const int id = tid + i * C::THREADS;
      const int row = id / C::CHUNKS_ROW, kc = id % C::CHUNKS_ROW;
      *(u32x4*)(&lds[buf][lds_off(row, kc)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) {
      const int id = tid + i * C::THREADS;
      const int row = id / C::CHUNKS_ROW, kc = id % C::CHUNKS_ROW;
      *(u32x4*)(&lds[buf][C::A_BYTES + lds_off(row, kc)]) = rb[i];
    }
  };

  // ---- scales: one dword per lane per 32-row tile per 256-wide k window ----------
  const int64_t a_bands = (p.a_rows + 31) / 32, b_bands = (p.b_rows + 31) / 32;
  auto load_scale = [&](const uint8_t* s, int64_t row0, int64_t bands, int64_t ktiles, int64_t kwin) -> unsigned {
    const int64_t band = row0 / 32;
    if (band >= bands) return 0x7f7f7f7fu;
    return *(const unsigned*)(s + scale_tile_base(band, kwin, ktiles) + 4 * l);
  };

  v16f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = (v16f){};

  const int64_t k_first = (k_beg / BK) * BK;
  const int64_t n_iter = k_end > k_beg ? (k_end - k_first + BK - 1) / BK : 0;

  if (n_iter > 0) {
    load_tile(k_first);
    store_tile(0);
  }
  __syncthreads();
  unsigned sa[C::TM], sb[C::TN];
  for (int64_t it = 0; it < n_iter; ++it) {
    const int buf = (int)(it & 1);
    const int64_t k0 = k_first + it * BK;
    if (it + 1 < n_iter) load_tile(k0 + BK);
    const int64_t kwin = k0 / 256;
    const int shift = (k0 & 255) ? 16 : 0;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      sa[i] = load_scale(p.a_s, a_row0 + wm * C::WM + 32 * i, a_bands, p.a_ktiles, kwin) >> shift;
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      sb[j] = load_scale(p.b_s, b_row0 + wn * C::WN + 32 * j, b_bands, p.b_ktiles, kwin) >> shift;

    const uint8_t* la = &lds[buf][0];
    const uint8_t* lb = &lds[buf][C::A_BYTES];
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      v8i fa[C::TM], fb[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int row = wm * C::WM + 32 * i + (l & 31);
        u32x4 lo = *(const u32x4*)(la + lds_off(row, 4 * s + h));
        u32x4 hi = *(const u32x4*)(la + lds_off(row, 4 * s + 2 + h));
        fa[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int row = wn * C::WN + 32 * j + (l & 31);
        u32x4 lo = *(const u32x4*)(lb + lds_off(row, 4 * s + h));
        u32x4 hi = *(const u32x4*)(lb + lds_off(row, 4 * s + 2 + h));
        fb[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          if (s == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, (int)sa[i], 0,
                                                                        (int)sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 1, (int)sa[i], 1,
                                                                        (int)sb[j]);
        }
    }
    if (it + 1 < n_iter) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------------------
  const int64_t row_limit = MODE == MODE_MGROUP ? a_row_end : p.M;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int64_t col = col0 + wn * C::WN + 32 * j + (l & 31);
      if (col >= n_limit) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = out_row0 + wm * C::WM + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row >= row_limit) continue;
        if (OUT_BF16)
          ((uint16_t*)out_base)[row * p.ldo + col] = f32_to_bf16_rne(acc[i][j][v]);
        else
          ((float*)out_base)[row * p.ldo + col] = acc[i][j][v];
      }
    }
}

}  // namespace mx

namespace {
constexpr int BM = 128, BN = 128, BK = 128, WAVES_M = 2, WAVES_N = 2;

template <int MODE>
hipError_t launch(mx::GemmArgs& p, int out_bf16, hipStream_t stream) {
  const int64_t blocks = MODE == mx::MODE_MGROUP ? p.mt_total * p.nt : (int64_t)p.groups * p.mt_total * p.nt;
  if (blocks == 0) return hipSuccess;
  const int threads = 64 * WAVES_M * WAVES_N;
  if (out_bf16)
    hipLaunchKernelGGL((mx::k_gemm<BM, BN, BK, WAVES_M, WAVES_N, MODE, 1>), dim3((unsigned)blocks), dim3(threads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((mx::k_gemm<BM, BN, BK, WAVES_M, WAVES_N, MODE, 0>), dim3((unsigned)blocks), dim3(threads), 0,
                       stream, p);
  return hipGetLastError();
}
}  // namespace

// M-grouped: C[m x n] = A[m x k] . B_g[n x k]^T per row group (forward and dgrad).
hipError_t mx_launch_gemm_mgroup(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                                 const int32_t* offs, int groups, int64_t m, int64_t n, int64_t k, void* out,
                                 int out_bf16, hipStream_t stream) {
  mx::GemmArgs p{};
  p.a = a; p.a_s = a_s; p.b = b; p.b_s = b_s; p.offs = offs; p.out = out;
  p.lda = k; p.ldb = k;
  p.a_rows = m; p.b_rows = (int64_t)groups * n;
  p.a_ktiles = p.b_ktiles = mx::scale_tiles_k(k / 32);
  p.M = m; p.N = n; p.K = k; p.ldo = n;
  p.groups = groups;
  p.mt_total = (m + BM - 1) / BM + (offs ? groups : 0);
  p.nt = (n + BN - 1) / BN;
  return launch<mx::MODE_MGROUP>(p, out_bf16, stream);
}

// K-grouped: C_g[m x n] = A[m x K_g] . B[n x K_g]^T over each group's contraction range (wgrad).
hipError_t mx_launch_gemm_kgroup(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                                 const int32_t* offs, int groups, int64_t m, int64_t n, int64_t k, void* out,
                                 int out_bf16, hipStream_t stream) {
  mx::GemmArgs p{};
  p.a = a; p.a_s = a_s; p.b = b; p.b_s = b_s; p.offs = offs; p.out = out;
  p.lda = k; p.ldb = k;
  p.a_rows = m; p.b_rows = n;
  p.a_ktiles = p.b_ktiles = mx::scale_tiles_k(k / 32);
  p.M = m; p.N = n; p.K = k; p.ldo = n;
  p.groups = groups;
  p.mt_total = (m + BM - 1) / BM;
  p.nt = (n + BN - 1) / BN;
  return launch<mx::MODE_KGROUP>(p, out_bf16, stream);
}
