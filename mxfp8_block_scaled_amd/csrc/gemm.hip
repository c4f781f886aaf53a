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
// 32x32 tile: lane l, register v -> row 8*(v/4) + 4*h + v%4 (of the first
// operand), column l % 32 (of the second). The kernel passes B first, so each
// lane accumulates four consecutive output columns of one output row per v/4:
// C[row l % 32][col 8*(v/4) + 4*h + v%4], which it stores directly.

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace mx {

enum { MODE_MGROUP = 0, MODE_KGROUP = 1 };
// Operand element kind: E4M3 codes with E8M0 block scales (the block-scaled MFMA),
// or plain bf16 (two bf16 MFMAs per 64-byte k-step, no scales).
enum { EL_MXFP8 = 0, EL_BF16 = 1 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct GemmArgs {
  const uint8_t* a;    // [a_rows x lda] codes
  const uint8_t* a_s;  // MFMA-blocked scales of a
  const uint8_t* b;
  const uint8_t* b_s;
  const int32_t* offs;  // device, may be null (one group)
  // M-grouped only, may be null: the groups' unpadded row ends when A's rows are the
  // token-group padded ones; the output is then written unpadded (row r of group g
  // at r - offs[g-1] + offs_out[g-1]) and the padding rows are not written
  const int32_t* offs_out;
  void* out;
  int64_t out_rows;  // M-grouped: rows of the output (M, or the unpadded rows with offs_out)
  int64_t lda, ldb;          // row pitch in bytes (= contraction length x element size)
  int64_t a_rows, b_rows;    // rows of the whole operand buffers
  int64_t a_ktiles, b_ktiles;  // scale tiles along the contraction
  int64_t M, N, K;  // M-grouped: M = token rows, N = per-group output columns, K = contraction
                    // K-grouped: M = rows of A, N = rows of B, K = contraction (tokens)
                    // (K and offs in elements; the kernel works in bytes of the contraction)
  int64_t ldo;      // output row pitch (elements)
  int64_t mt_total, nt;  // tile grid: m-tiles (upper bound for M-grouped), n-tiles
  int64_t tiles;         // logical tiles (some M-grouped ones may be empty)
  int groups;
  int splits;            // K-grouped: contraction splits (1 = none), partials in fp32 at out
  int64_t split_stride;  // elements between the partial outputs of consecutive splits
  int tail;              // M-grouped with offs: TAIL_NONE, TAIL_MAIN or TAIL_SUB (below)
};

// The last, partial round of an M-grouped launch with offs. The real tile count is
// known only on the device, so the split is decided there: with TAIL_MAIN the
// 256x256 launch runs only each XCD's whole rounds (one tile per compute unit each)
// when at most half a round is left over, and a second launch of 128x128 tiles
// (TAIL_SUB) runs each XCD's left-over tiles as four quarters each, on the same XCD
// and on four times as many compute units.
enum { TAIL_NONE = 0, TAIL_MAIN = 1, TAIL_SUB = 2 };

// Block tile BM x BN over a WGM x WGN grid of waves, each wave (BM/WGM) x (BN/WGN)
// in 32x32 MFMA tiles; the contraction advances 64 elements (one MFMA k-step) per
// pipeline stage, over a ring of NST stages in LDS.
template <int BM, int BN, int WGM, int WGN, int NST_>
struct Cfg {
  static constexpr int WAVES = WGM * WGN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BK = 64;
  static constexpr int NST = NST_;  // LDS ring depth: NST - 1 stages are loaded ahead
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  // scale tiles of one 256-wide window: A's bands, then B's, 256 B each, each side
  // in a whole number of 1 KB slots (four bands; a slot past the side's last band
  // holds scales of rows outside the tile, never read); two windows are resident
  // (the one in use and the next)
  static constexpr int A_SLOTS = (BM / 32 + 3) / 4 * 4, B_SLOTS = (BN / 32 + 3) / 4 * 4;
  static constexpr int BANDS = A_SLOTS + B_SLOTS;
  static constexpr int SC_BYTES = WAVES * 1024;  // 1 KB per wave; waves past BANDS/4 fill theirs with zeros
  static constexpr int LDS_BYTES = NST * STAGE_BYTES + 2 * SC_BYTES;
  // per wave and stage: its share of A and B rows in 1 KB loads (16 rows x 64 B);
  // per window: one 1 KB load (four 256-byte scale tiles) by every wave (out of
  // range, i.e. zeros, for waves past SC_WAVES, so every wave issues the same loads)
  static constexpr int A_ROWS_W = BM / WAVES, B_ROWS_W = BN / WAVES;
  static constexpr int A_LOADS = A_ROWS_W / 16, B_LOADS = B_ROWS_W / 16;
  static constexpr int AB_LOADS = A_LOADS + B_LOADS;
  static constexpr int SC_WAVES = BANDS / 4;
  // rows of a wave's 32x32 tiles whose MFMAs run before the pipeline's wait and
  // barrier: three quarters where the rows split so (more matrix work in flight
  // while the wave waits), else half; the rest run beside the next step's LDS reads
  static constexpr int HEAD_ROWS = TM % 4 == 0 ? TM * 3 / 4 : TM / 2;
  static constexpr int TAIL_MFMAS = (TM - HEAD_ROWS) * TN;
  static_assert(SC_WAVES <= WAVES && A_ROWS_W % 16 == 0 && B_ROWS_W % 16 == 0, "tile shape");
  static_assert(TM % 2 == 0 && 2 * AB_LOADS + 2 < 64 && NST >= 2 && NST <= 4, "");
};

// LDS holds each 64-byte row (four 16-byte chunks of one k-step) with chunk c of
// row r at slot c ^ ((r >> 2) & 3): sixteen consecutive rows reading the same chunk
// then hit sixteen different 16-byte bank groups.

// Rows per epilogue staging pass: the largest multiple of 32 that divides the wave's
// rows `wm` and fits `cap` rows of staging.
constexpr int epi_rows(int wm, int cap) {
  int r = wm;
  while (r > 32 && (r > cap || wm % r != 0)) r -= 32;
  return r;
}

__device__ inline int32_t group_start(const int32_t* offs, int g) { return g == 0 ? 0 : offs[g - 1]; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define MX_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One output tile: where it sits and what it contracts over.
struct Tile {
  int64_t a_row0, a_row_end, b_row0, b_row_end, k_beg, k_end, col0;
  int64_t out_limit, out_shift;  // M-grouped: output rows [a_row0, out_limit) go to row + out_shift
  uint8_t* out_base;
  bool valid;
};

// The group owning m-tile `mt` of the concatenated per-group m-tile lists (M-grouped):
// row range [s, e) of the group and, for padded outputs, its output range [so, eo).
struct GroupHit {
  int64_t s, e, so, eo, cum;  // cum: m-tiles of the groups before it
  int g;                      // -1: no group owns mt
};

// Inclusive scans over the 64 lanes of a wave of values >= 0 (0 is the identity of
// both), in DPP moves between lanes: four row shifts give the scan inside each row of
// 16 lanes, then the last lane of row 0 (of row 2) is added into row 1 (row 3) and the
// last lane of row 1 into rows 2 and 3. Each step is one ALU operation on a
// neighbour's register, where a shuffle through LDS costs a round trip per step.
__device__ inline int32_t dpp_max_step(int32_t v, int32_t w) { return w > v ? w : v; }
template <bool MAX>
__device__ inline int32_t wave_incl_scan(int32_t v) {
  auto op = [](int32_t a, int32_t b) { return MAX ? dpp_max_step(a, b) : a + b; };
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));  // row_bcast:15 into rows 1, 3
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));  // row_bcast:31 into rows 2, 3
  return v;
}
// The value of the previous lane (lane 0: `first`).
__device__ inline int32_t wave_prev(int32_t v, int32_t first) {
  return __builtin_amdgcn_update_dpp(first, v, 0x138, 0xf, 0xf, false);  // wave_shr:1
}

// Groups g0 .. g0+63 of the M-grouped scan, lane l holding group g0 + l: its row
// range [s, e), output range [so, eo), m-tiles, and the m-tiles of all groups up to
// and including it. The ends are read clamped into [0, M] (the output ends into
// [0, out_rows]) as their running maximum: for valid offs this changes nothing; an
// out-of-contract offs gives wrong rows but no access outside the operand and output
// buffers. Lanes past the last group hold an empty range and the running totals.
// Everything fits 32 bits: offs are int32 and the m-tile counts are below 2^27.
struct GroupChunk {
  int32_t s, e, so, eo, tiles, cum;
  bool live;
};

template <int BM>
__device__ inline GroupChunk scan_chunk(const GemmArgs& p, int g0, int32_t carry_e, int32_t carry_eo,
                                        int32_t carry_cum) {
  const int l = threadIdx.x & 63;
  const int g = g0 + l;
  const int32_t m32 = p.M < INT32_MAX ? (int32_t)p.M : INT32_MAX;
  const int32_t o32 = p.out_rows < INT32_MAX ? (int32_t)p.out_rows : INT32_MAX;
  GroupChunk c;
  c.live = g < p.groups;
  int32_t e = c.live ? p.offs[g] : 0, eo = c.live && p.offs_out ? p.offs_out[g] : 0;
  e = e < 0 ? 0 : (e > m32 ? m32 : e);
  eo = eo < 0 ? 0 : (eo > o32 ? o32 : eo);
  e = wave_incl_scan<true>(e > carry_e ? e : carry_e);
  eo = wave_incl_scan<true>(eo > carry_eo ? eo : carry_eo);
  c.s = wave_prev(e, carry_e);
  c.so = wave_prev(eo, carry_eo);
  c.e = e;
  c.eo = eo;
  c.tiles = c.live ? (e - c.s + BM - 1) / BM : 0;
  c.cum = wave_incl_scan<false>(c.tiles) + carry_cum;
  return c;
}

// The m-tiles of all groups (the first chunk's scan is kept in `first`). Every wave
// scans on its own, 64 groups per step: no LDS, no barrier, and a thousand groups
// cost a few dozen steps where a group-by-group walk would wait on one load per group.
template <int BM>
__device__ inline int64_t total_mtiles(const GemmArgs& p, GroupChunk& first) {
  first = scan_chunk<BM>(p, 0, 0, 0, 0);
  int32_t ce = __builtin_amdgcn_readlane(first.e, 63), ceo = __builtin_amdgcn_readlane(first.eo, 63);
  int32_t cc = __builtin_amdgcn_readlane(first.cum, 63);
  for (int g0 = 64; g0 < p.groups; g0 += 64) {
    const GroupChunk c = scan_chunk<BM>(p, g0, ce, ceo, cc);
    ce = __builtin_amdgcn_readlane(c.e, 63);
    ceo = __builtin_amdgcn_readlane(c.eo, 63);
    cc = __builtin_amdgcn_readlane(c.cum, 63);
  }
  return cc;
}

// The group owning m-tile `mt`: a ballot over each chunk, starting from the first.
template <int BM>
__device__ inline GroupHit find_group(const GemmArgs& p, int64_t mt, const GroupChunk& first) {
  GroupChunk c = first;
  for (int g0 = 0;;) {
    const uint64_t own = __ballot(c.live && mt >= c.cum - c.tiles && mt < c.cum);
    if (own) {
      const int j = __builtin_amdgcn_readfirstlane(__ffsll((long long)own) - 1);
      return GroupHit{__builtin_amdgcn_readlane(c.s, j), __builtin_amdgcn_readlane(c.e, j),
                      __builtin_amdgcn_readlane(c.so, j), __builtin_amdgcn_readlane(c.eo, j),
                      __builtin_amdgcn_readlane(c.cum - c.tiles, j), g0 + j};
    }
    g0 += 64;
    if (g0 >= p.groups) return GroupHit{0, 0, 0, 0, 0, -1};
    c = scan_chunk<BM>(p, g0, __builtin_amdgcn_readlane(c.e, 63), __builtin_amdgcn_readlane(c.eo, 63),
                       __builtin_amdgcn_readlane(c.cum, 63));
  }
}

// a / b and a % b for a, b >= 0: a 32-bit division when both fit (a few instructions
// where a 64-bit one is a long expansion), else the 64-bit one.
__device__ inline int64_t udiv(int64_t a, int64_t b) {
  return ((a | b) >> 32) == 0 ? (int64_t)((uint32_t)a / (uint32_t)b) : a / b;
}
__device__ inline int64_t umod(int64_t a, int64_t b) { return a - udiv(a, b) * b; }

// Logical tile t -> its output tile and contraction range (one block per tile).
// Each XCD takes a contiguous range of logical tiles in order (xcd_remap,
// spread_tiles); with a raster, over `mt_count` m-tiles, of bands of GM m-tiles by all n-tiles,
// the ~32 tiles in flight on one XCD share their A and B slices in its L2 (GM = 4
// measured best among 1..16).
template <int BM, int BN, int MODE, int OUT_BF16, int EL>
__device__ inline Tile tile_at(const GemmArgs& p, int64_t t, int64_t mt_count, const GroupChunk& first) {
  constexpr int64_t GM = 4;
  constexpr int64_t EB = EL == EL_BF16 ? 2 : 1;  // bytes per contraction element
  constexpr int out_es = OUT_BF16 ? 2 : 4;
  Tile T{};
  T.out_base = (uint8_t*)p.out;
  const int64_t per_g = p.mt_total * p.nt;
  int64_t r = t;
  int g = 0;
  int sp = 0;  // contraction split (K-grouped only)
  if (MODE == MODE_KGROUP) {
    sp = (int)(t / (p.groups * per_g));
    t -= (int64_t)sp * p.groups * per_g;
    // slice-major: each group's raster is cut into 8 slices of S tiles and the
    // order runs slice by slice, every group's slice s (in group order) before
    // slice s+1. The XCD remap hands XCD x about the x-th eighth of the order, i.e.
    // slice x of every group, so the XCDs share each group's (uneven) contraction
    // length evenly. (Starting slice s at group s instead, so that the XCDs worked
    // on different groups at once, ran 1-4% slower on the 8-expert and 32-expert
    // wgrads; so did taking the groups largest first.)
    const int64_t S = (per_g + 7) / 8;
    const int64_t G = p.groups;
    const int64_t sl = t / (G * S);
    const int64_t n_s = per_g - sl * S < S ? per_g - sl * S : S;  // tiles in this slice
    const int64_t rem = t - sl * G * S;
    g = (int)(rem / n_s);
    r = sl * S + rem % n_s;
  }
  const int64_t band = udiv(r, GM * p.nt);
  const int64_t first_m = band * GM;
  const int64_t gm = mt_count - first_m < GM ? mt_count - first_m : GM;
  const int64_t in_band = r - band * GM * p.nt;
  const int64_t mt = first_m + (gm == GM ? in_band % GM : umod(in_band, gm));
  const int64_t n_tile = gm == GM ? in_band / GM : udiv(in_band, gm);
  T.col0 = n_tile * BN;
  if (MODE == MODE_MGROUP) {
    // the group owning m-tile `mt` (dense: the one group of all M rows)
    GroupHit hit{0, p.M, 0, p.out_rows, 0, 0};
    if (p.offs) hit = find_group<BM>(p, mt, first);
    const int found = hit.g;
    if (found >= 0) {
      T.a_row0 = hit.s + (mt - hit.cum) * BM;
      T.a_row_end = hit.e;
      T.out_limit = hit.e;
      if (p.offs_out) {
        const int64_t real_end = hit.s + (hit.eo - hit.so);  // the group's real rows, padded coordinates
        T.out_shift = hit.so - hit.s;
        T.out_limit = real_end < hit.e ? real_end : hit.e;
      }
    }
    T.valid = found >= 0;
    g = found < 0 ? 0 : found;
    T.b_row0 = (int64_t)g * p.N + n_tile * BN;
    T.b_row_end = (int64_t)g * p.N + p.N;
    T.k_beg = 0;
    T.k_end = p.K * EB;
  } else {
    T.valid = true;
    T.a_row0 = mt * BM;
    T.a_row_end = p.M;
    T.b_row0 = n_tile * BN;
    T.b_row_end = p.N;
    // the group's token range clamped into [0, K] (out-of-contract offs: wrong sums,
    // no access outside the operands)
    int64_t kb = p.offs ? group_start(p.offs, g) : 0, ke = p.offs ? p.offs[g] : p.K;
    kb = kb < 0 ? 0 : (kb > p.K ? p.K : kb);
    ke = ke < kb ? kb : (ke > p.K ? p.K : ke);
    T.k_beg = EB * kb;
    T.k_end = EB * ke;
    if (p.splits > 1) {
      // split sp of `splits` takes a run of whole 256-wide windows (counted from the
      // 256-aligned start of the group's range), so no split adds masked steps; it
      // writes an fp32 partial, summed afterwards in split order
      const int64_t k0 = (T.k_beg / 256) * 256;
      const int64_t wins = T.k_end > T.k_beg ? (T.k_end - k0 + 255) / 256 : 0;
      const int64_t w0 = wins * sp / p.splits, w1 = wins * (sp + 1) / p.splits;
      const int64_t nb = k0 + 256 * w0 > T.k_beg ? k0 + 256 * w0 : T.k_beg;
      const int64_t ne = k0 + 256 * w1 < T.k_end ? k0 + 256 * w1 : T.k_end;
      T.k_beg = nb;
      T.k_end = ne > nb ? ne : nb;
      T.out_base += (int64_t)sp * p.split_stride * out_es;
    }
    T.out_base += (int64_t)g * p.M * p.ldo * out_es;
  }
  return T;
}

// A block-uniform value computed in vector registers (a 64-bit division, a load
// through a vector address) is not known to be uniform; reading lane 0 makes it a
// scalar again, so buffer offsets and descriptors built from it need no per-lane loop.
__device__ inline int64_t uniform(int64_t v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Tile order: blocks are dealt round-robin to the 8 XCDs, so the remap gives each
// XCD a contiguous range of logical tiles; with the GM-band raster of tile_at, the
// ~32 tiles resident on one XCD share their A and B slices in its L2.
__device__ inline int64_t xcd_remap(int64_t bid, int64_t nblk) {
  const int64_t per_xcd = nblk / 8;
  return bid < per_xcd * 8 ? (bid % 8) * per_xcd + bid / 8 : bid;
}

// The same for `real` tiles on a grid of nblk >= real blocks (M-grouped with offs:
// the grid is sized for the most m-tiles any group split can need, the real count is
// known only on the device): XCD x takes [x * per, (x+1) * per) with per = real / 8
// rounded up, so every XCD gets an eighth of the real work. Dividing the grid instead
// left the unused blocks all at the end, on the last XCD: at the MoE step's 1088 real
// tiles of 1152, XCDs 0-6 ran 144 tiles (4.5 rounds of 32 compute units) and XCD 7
// ran 80. -1: the block has no tile.
__device__ inline int64_t spread_tiles(int64_t bid, int64_t nblk, int64_t real) {
  const int64_t nx = nblk / 8, per = (real + 7) / 8;
  if (per <= nx) {
    const int64_t j = bid / 8, t = (bid % 8) * per + j;
    return bid < nx * 8 && j < per && t < real ? t : -1;
  }
  const int64_t t = xcd_remap(bid, nblk);
  return t < real ? t : -1;
}

// The XCD shares of `real` 256x256 tiles with a TAIL_MAIN / TAIL_SUB pair: XCD x
// owns tiles [x * per, (x+1) * per), per = real / 8 rounded up (as spread_tiles deals
// them); TAIL_MAIN runs the first `mainp` of them (whole rounds of the XCD's 32
// compute units) and TAIL_SUB the `restp` after them as quarters, when 1..16 are left
// (two quarters per compute unit at most); otherwise restp = 0 and TAIL_MAIN runs all.
// Keeping every tile on the XCD that spread_tiles gives it keeps the XCDs at different
// places of the raster at once: a split that gave each XCD whole bands (all of them
// starting on the same columns of their groups' B) ran the dgrad inside the training
// step 3 us slower, not faster.
struct TailSplit {
  int64_t per, mainp, restp;
};
__device__ inline TailSplit tail_split(int64_t real) {
  TailSplit s;
  s.per = (real + 7) / 8;
  s.mainp = s.per / 32 * 32;
  s.restp = s.per - s.mainp;
  if (!(s.mainp > 0 && s.restp > 0 && s.restp <= 16)) {
    s.mainp = s.per;
    s.restp = 0;
  }
  return s;
}

// WPE: waves per SIMD the register allocation must allow (2 where two blocks
// share a compute unit).
#ifdef MX_CYCLE_STAMPS
// Instrumented build only (libmxfp8_stamps.so): wave 0 of every block records the
// shader clock (s_memtime) at its start, when the first stage has landed, when the
// last k-step is done and after the epilogue's stores are issued, with the hardware
// ids of its compute unit and the tile's k-steps. 8 words per block; the second
// launch of a split last round (128x128 quarters) records at kStampBlocks / 2 on.
constexpr int64_t kStampBlocks = 32768;
__device__ unsigned long long g_cycle_stamps[kStampBlocks * 8];
#endif

template <int BM, int BN, int WGM, int WGN, int NST_, int WPE, int MODE, int OUT_BF16, int EL>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(WPE))) void k_gemm(GemmArgs p) {
  using C = Cfg<BM, BN, WGM, WGN, NST_>;
  constexpr int NST = C::NST, BK = C::BK;
  constexpr bool SCALED = EL == EL_MXFP8;
  constexpr int MPK = SCALED ? 1 : 2;  // MFMAs per 32x32 tile and 64-byte k-step
  // LDS reads per k-step (two 16-byte fragment halves per tile, plus one scale dword
  // per tile when scaled) spread over the tail MFMAs
  constexpr int DS_PER_MFMA = ((SCALED ? 3 : 2) * (C::TM + C::TN) + C::TAIL_MFMAS - 1) / C::TAIL_MFMAS;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
#ifdef MX_CYCLE_STAMPS
  const unsigned long long st_t0 = __builtin_amdgcn_s_memtime(), st_rt = __builtin_amdgcn_s_memrealtime();
  unsigned long long st_t1 = 0, st_t2 = 0;
#endif

  const int tid = threadIdx.x, l = tid & 63, h = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / WGN, wn = wave % WGN;
  GroupChunk first{};
  int64_t mt_count = p.mt_total, t;
  Tile T;
  constexpr bool QUARTERS = MODE == MODE_MGROUP && BM == 128 && BN == 128;
  if (QUARTERS && p.offs && p.tail == TAIL_SUB) {
    if constexpr (QUARTERS) {
      // block j of XCD x (blocks reach XCDs round-robin): quarter j % 4 (row half,
      // column half) of the XCD's left-over tile j / 4 in the 256x256 geometry
      mt_count = uniform(total_mtiles<2 * BM>(p, first));
      GemmArgs pp = p;
      pp.nt = (p.N + 2 * BN - 1) / (2 * BN);
      const int64_t real = mt_count * pp.nt;
      const TailSplit sp = tail_split(real);
      const int64_t x = blockIdx.x % 8, j = blockIdx.x / 8;
      if (sp.restp == 0 || j >= sp.restp * 4) return;
      const int64_t tt = x * sp.per + sp.mainp + j / 4;
      if (tt >= real) return;
      T = tile_at<2 * BM, 2 * BN, MODE, OUT_BF16, EL>(pp, tt, mt_count, first);
      const int q = (int)(j & 3);
      T.a_row0 += (q >> 1) * BM;
      T.col0 += (q & 1) * BN;
      T.b_row0 += (q & 1) * BN;
      if (T.a_row0 >= T.a_row_end || T.col0 >= p.N) T.valid = false;
    }
  } else {
    if (MODE == MODE_MGROUP && p.offs) {
      mt_count = uniform(total_mtiles<BM>(p, first));
      const int64_t real = mt_count * p.nt;
      const TailSplit sp = tail_split(real);
      if (p.tail == TAIL_MAIN && sp.restp > 0) {
        // the first mainp tiles of each XCD's share (mainp <= real / 8 <= grid / 8)
        const int64_t x = blockIdx.x % 8, j = blockIdx.x / 8;
        t = j < sp.mainp && x * sp.per + j < real ? x * sp.per + j : -1;
      } else {
        t = spread_tiles(blockIdx.x, gridDim.x, real);
      }
      t = uniform(t);
      if (t < 0) return;
    } else {
      t = xcd_remap(blockIdx.x, gridDim.x);
    }
    T = tile_at<BM, BN, MODE, OUT_BF16, EL>(p, t, mt_count, first);
  }
  if (!__builtin_amdgcn_readfirstlane((int)T.valid)) return;
  T.a_row0 = uniform(T.a_row0); T.a_row_end = uniform(T.a_row_end);
  T.b_row0 = uniform(T.b_row0); T.b_row_end = uniform(T.b_row_end);
  T.k_beg = uniform(T.k_beg); T.k_end = uniform(T.k_end); T.col0 = uniform(T.col0);
  T.out_base = (uint8_t*)uniform((int64_t)T.out_base);
  T.out_limit = uniform(T.out_limit); T.out_shift = uniform(T.out_shift);

  const int64_t a_bands = (p.a_rows + 31) / 32, b_bands = (p.b_rows + 31) / 32;
  const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.a_s, (short)0, (int)(a_bands * p.a_ktiles * 256), 0x00020000);
  const __amdgpu_buffer_rsrc_t bs_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.b_s, (short)0, (int)(b_bands * p.b_ktiles * 256), 0x00020000);
  const int kc_l = (l & 3) ^ (l >> 4);
  const int a_row_l = wave * C::A_ROWS_W + (l >> 2), b_row_l = wave * C::B_ROWS_W + (l >> 2);
  // Per-lane offsets are fixed for a tile (row and chunk); the contraction position
  // goes in the scalar offset. Lanes whose chunk lies outside [k_beg, k_end) in a
  // given stage switch to an out-of-range offset, which reads as zero.
  const unsigned a_off0 = (unsigned)(a_row_l * p.lda + kc_l * 16), a_offq = (unsigned)(16 * p.lda);
  const unsigned b_off0 = (unsigned)(b_row_l * p.ldb + kc_l * 16), b_offq = (unsigned)(16 * p.ldb);
  const int sc_band = wave * 4 + (l >> 4);  // index in the A-then-B band list
  const bool sc_is_a = wave < C::A_SLOTS / 4;  // A's slots come first, whole waves each

  // contraction steps of BK from the 256-aligned position at or below k_beg (a scale
  // window boundary: every fourth stage opens a window; stages before k_beg are
  // masked to zero)
  const int64_t k_first = (T.k_beg / 256) * 256;
  const int64_t n_iter = T.k_end > T.k_beg ? (T.k_end - k_first + BK - 1) / BK : 0;
  const int kb32 = (int)T.k_beg, ke32 = (int)T.k_end;  // contraction lengths are < 2^31
  // Raw buffer descriptors span exactly the valid rows of the tile, so rows past the
  // group / matrix end read as zero.
  const int64_t a_lim = T.a_row_end < p.a_rows ? T.a_row_end : p.a_rows;
  const int64_t b_lim = T.b_row_end < p.b_rows ? T.b_row_end : p.b_rows;
  const int64_t a_valid = a_lim > T.a_row0 ? (a_lim - T.a_row0 < BM ? a_lim - T.a_row0 : BM) : 0;
  const int64_t b_valid = b_lim > T.b_row0 ? (b_lim - T.b_row0 < BN ? b_lim - T.b_row0 : BN) : 0;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + T.a_row0 * p.lda), (short)0, (int)(a_valid * p.lda), 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.b + T.b_row0 * p.ldb), (short)0, (int)(b_valid * p.ldb), 0x00020000);
  const int64_t sc_row_band = sc_is_a ? T.a_row0 / 32 + sc_band : T.b_row0 / 32 + (sc_band - C::A_SLOTS);
  const int64_t sc_ktiles = sc_is_a ? p.a_ktiles : p.b_ktiles;
  const unsigned sc_off = wave < C::SC_WAVES && sc_row_band < (sc_is_a ? a_bands : b_bands)
                              ? (unsigned)(sc_row_band * sc_ktiles * 256 + (l & 15) * 16)
                              : 0x80000000u;

  // Every step issues the A/B loads of one stage (C::AB_LOADS per wave) plus, when
  // that stage opens a 256-wide scale window, one scale load by each of the first
  // C::SC_WAVES waves. A stage past the end of the contraction (`live` false)
  // issues the same loads out of range: they read nothing and only fill LDS that is
  // never consumed, so the counter arithmetic is the same on every step.
  // k_first is 256-aligned, so stage s opens a scale window iff s % 4 == 0; callers
  // pass s % 4 as a compile-time constant where they can (the unrolled steps)
  auto issue_stage = [&](int64_t s_idx, int s_mod4, bool live) {
    const int64_t k0 = k_first + s_idx * BK;
    uint8_t* st = lds + ((int)s_idx % NST) * C::STAGE_BYTES;
    const int kk = (int)k0 + kc_l * 16;
    // this lane's chunk is masked; in bf16 a group edge may fall inside a 16-byte
    // chunk (8 tokens): such chunks are loaded and their outside elements zeroed in
    // the fragment registers (read_frags)
    const bool drop = !live || (SCALED ? kk < kb32 : kk + 16 <= kb32) || kk >= ke32;
    const int soff = live ? (int)k0 : 0;
#pragma unroll
    for (int q = 0; q < C::A_LOADS; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(st + wave * C::A_ROWS_W * 64 + q * 1024), 16,
                                               drop ? 0x80000000u : a_off0 + q * a_offq, soff, 0, 0);
#pragma unroll
    for (int q = 0; q < C::B_LOADS; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr_t)(st + C::A_BYTES + wave * C::B_ROWS_W * 64 + q * 1024),
                                               16, drop ? 0x80000000u : b_off0 + q * b_offq, soff, 0, 0);
    if (SCALED && s_mod4 == 0) {
      const int64_t kwin = k0 / 256;
      uint8_t* dst = lds + NST * C::STAGE_BYTES + (int)(kwin & 1) * C::SC_BYTES + wave * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sc_is_a ? as_rsrc : bs_rsrc, (lds_ptr_t)dst, 16,
                                               live ? sc_off : 0x80000000u, live ? (int)(kwin * 256) : 0, 0, 0);
    }
  };
  // loads this wave issues for the `count` stages following a stage with s % 4 == s_mod4
  auto loads_after = [&](int s_mod4, int count) -> int {
    int n = 0;
    for (int q = 1; q <= count; ++q) n += C::AB_LOADS + ((SCALED && ((s_mod4 + q) & 3) == 0) ? 1 : 0);
    return n;
  };
  auto wait_n = [&](int n) {  // s_waitcnt needs an immediate; n takes one of a few values
    if (n >= 2 * C::AB_LOADS + 1) MX_WAIT_VMCNT(2 * C::AB_LOADS + 1);
    else if (n == 2 * C::AB_LOADS) MX_WAIT_VMCNT(2 * C::AB_LOADS);
    else if (n == C::AB_LOADS + 1) MX_WAIT_VMCNT(C::AB_LOADS + 1);
    else if (n == C::AB_LOADS) MX_WAIT_VMCNT(C::AB_LOADS);
    else MX_WAIT_VMCNT(0);
  };

  // ---- fragments: lane reads chunks h and h+2 of its row (32 bytes) ---------------
  const int frow = l & 31;
  const int sw = (frow >> 2) & 3;
  const int off_lo = frow * 64 + ((h ^ sw) << 4), off_hi = frow * 64 + (((h + 2) ^ sw) << 4);
  struct Frag {
    v8i a[C::TM], b[C::TN];
    unsigned sa[C::TM], sb[C::TN];
  };
  // `masked` (a compile-time flag): the tile's contraction range cuts a 16-byte chunk
  auto read_frags = [&](Frag& f, int buf, int64_t k0, auto masked) {
    const uint8_t* st = lds + buf * C::STAGE_BYTES;
    const uint8_t* sc = lds + NST * C::STAGE_BYTES + (int)((k0 >> 8) & 1) * C::SC_BYTES;
    const uint8_t* la = st + wm * C::WM * 64;
    const uint8_t* lb = st + C::A_BYTES + wn * C::WN * 64;
    const int sh = (int)((k0 >> 6) & 3) * 8;  // byte of the window dword for this k-step
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      u32x4 lo = *(const u32x4*)(lb + j * 2048 + off_lo);
      u32x4 hi = *(const u32x4*)(lb + j * 2048 + off_hi);
      f.b[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      if (SCALED) f.sb[j] = *(const unsigned*)(sc + (C::A_SLOTS + wn * C::TN + j) * 256 + 4 * l) >> sh;
    }
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      u32x4 lo = *(const u32x4*)(la + i * 2048 + off_lo);
      u32x4 hi = *(const u32x4*)(la + i * 2048 + off_hi);
      f.a[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      if (SCALED) f.sa[i] = *(const unsigned*)(sc + (wm * C::TM + i) * 256 + 4 * l) >> sh;
    }
    if constexpr (decltype(masked)::value) {
      // a k-step that a group edge cuts: zero A's elements outside [k_beg, k_end)
      // (A alone suffices: the products with them vanish)
      const int kb = (int)k0;
      if (kb < kb32 || kb + BK > ke32) {
        int mk[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const int byte = kb + (d < 4 ? 16 * h + 4 * d : 32 + 16 * h + 4 * (d - 4));
          mk[d] = (byte >= kb32 && byte < ke32 ? 0xFFFF : 0) | (byte + 2 >= kb32 && byte + 2 < ke32 ? (int)0xFFFF0000 : 0);
        }
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int d = 0; d < 8; ++d) f.a[i][d] &= mk[d];
      }
    }
  };

  v16f acc[C::TM][C::TN];
  auto mfma_rows = [&](const Frag& f, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        if (SCALED) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], 0, 0, 0,
                                                                      (int)f.sb[j], 0, (int)f.sa[i]);
        } else {
          // the lane's two 16-byte halves are the two 16-element k-slices of the step
          const v8i bj = f.b[j], ai = f.a[i];
          const bf16x8 b_lo = __builtin_bit_cast(bf16x8, (u32x4){(unsigned)bj[0], (unsigned)bj[1], (unsigned)bj[2], (unsigned)bj[3]});
          const bf16x8 b_hi = __builtin_bit_cast(bf16x8, (u32x4){(unsigned)bj[4], (unsigned)bj[5], (unsigned)bj[6], (unsigned)bj[7]});
          const bf16x8 a_lo = __builtin_bit_cast(bf16x8, (u32x4){(unsigned)ai[0], (unsigned)ai[1], (unsigned)ai[2], (unsigned)ai[3]});
          const bf16x8 a_hi = __builtin_bit_cast(bf16x8, (u32x4){(unsigned)ai[4], (unsigned)ai[5], (unsigned)ai[6], (unsigned)ai[7]});
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_lo, a_lo, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_hi, a_hi, acc[i][j], 0, 0, 0);
        }
  };

  // One pipeline step over an NST-deep LDS ring. Step `it` issues stage it+NST-1,
  // runs the MFMAs of stage it's first HEAD_ROWS tile rows, waits for its own loads of stage it+1
  // (at most NST-2 later stages stay in flight), meets the other waves at a barrier
  // (so stage it+1 is complete in LDS and every wave is past stage it-1, whose slot
  // the next issue overwrites), then reads stage it+1's fragments interleaved with
  // the remaining rows' MFMAs. `s4` is it % 4 (a constant in the unrolled
  // loop): it places the scale windows, and the ring slots for NST 2 and 4.
  auto step = [&](int64_t it, int s4, const Frag& cur, Frag& nxt, auto masked) {
    const int slot = s4;
    issue_stage(it + NST - 1, (slot + NST - 1) & 3, it + NST - 1 < n_iter);
    mfma_rows(cur, 0, C::HEAD_ROWS);
    // spread the loads over the MFMAs so no load waits in front of an idle matrix core
#pragma unroll
    for (int q = 0; q < C::HEAD_ROWS * C::TN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, MPK, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU (load offsets)
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_n(loads_after((slot + 1) & 3, NST - 2));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(nxt, NST == 3 ? (int)(it + 1) % 3 : (slot + 1) % NST, k_first + (it + 1) * BK, masked);
    mfma_rows(cur, C::HEAD_ROWS, C::TM);
    // interleave: one MFMA, then a share of the LDS reads
#pragma unroll
    for (int q = 0; q < C::TAIL_MFMAS; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, MPK, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, DS_PER_MFMA, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- epilogue ------------------------------------------------------------------
  // Each lane holds four consecutive columns of one row per v/4. In the common case
  // (the wave's columns inside N, rows 16-byte aligned) each wave stages its WM x WN
  // output in its share of the idle ring, in passes of RP rows where the share holds
  // fewer (fp32 at 256x256: two): 8- or 16-byte LDS writes, 16-byte chunks of a row
  // XOR-swizzled by the row
  // so neither the writes (32 rows, one chunk) nor the reads (whole rows) collide in
  // banks. It then writes whole row segments (WN * ES bytes) with 16-byte stores.
  // Otherwise (the ragged right edge) lanes store elements with a bounds check.
  auto epilogue = [&]() {
    const int64_t row_limit = MODE == MODE_MGROUP ? T.out_limit : p.M;
    const int64_t row_shift = MODE == MODE_MGROUP ? T.out_shift : 0;
    constexpr int ES = OUT_BF16 ? 2 : 4;
    constexpr int ROW_BYTES = C::WN * ES;
    constexpr int CPR = ROW_BYTES / 16;                      // 16-byte chunks per row
    // rows of a power-of-two number of chunks are XOR-swizzled in place; others (96-
    // column waves: 12 or 24 chunks) get one spare chunk per row, an odd pitch in
    // chunks, so 32 rows at one column spread over the banks
    constexpr bool POW2 = (CPR & (CPR - 1)) == 0;
    constexpr int PITCH = POW2 ? ROW_BYTES : ROW_BYTES + 16;
    constexpr int EPI_BYTES = NST * C::STAGE_BYTES / C::WAVES;  // staging bytes per wave
    constexpr int RP = epi_rows(C::WM, EPI_BYTES / PITCH);   // rows per pass
    constexpr int READS = RP * CPR / 64;                     // 16-byte reads / stores per lane and pass
    static_assert(CPR <= 64 && RP * CPR % 64 == 0, "rows of whole 16-byte chunks");
    static_assert(RP * PITCH <= EPI_BYTES && C::WM % RP == 0, "epilogue staging shape");
    const int64_t wrow0 = T.a_row0 + wm * C::WM;
    const int64_t wcol0 = T.col0 + wn * C::WN;
    if (((p.ldo * ES) & 15) == 0 && wcol0 + C::WN <= p.N) {
      uint8_t* stg = lds + wave * EPI_BYTES;
#pragma unroll
      for (int pass = 0; pass < C::WM / RP; ++pass) {
#pragma unroll
        for (int ii = 0; ii < RP / 32; ++ii) {
          const int i = pass * (RP / 32) + ii;
          const int r = 32 * ii + (l & 31);
          uint8_t* srow = stg + r * PITCH;
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int lb = (32 * j + 8 * q + 4 * h) * ES;  // byte of the lane's first column
              uint8_t* dst = srow + (POW2 ? ((((lb >> 4) ^ r) & (CPR - 1)) << 4) + (lb & 15) : lb);
              const v16f& c = acc[i][j];
              if (OUT_BF16)
                *(u32x2*)dst = (u32x2){bf16x2_rne(c[4 * q], c[4 * q + 1]), bf16x2_rne(c[4 * q + 2], c[4 * q + 3])};
              else
                *(v4f*)dst = (v4f){c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]};
            }
        }
// bf16 rows: fully unrolled; fp32 (two staging passes): by 4, as the full
        // unroll keeps too many read-back loads in flight beside the accumulators
        // still live for the second pass and spills
        constexpr int EPI_UNROLL = OUT_BF16 ? READS : 4;
#pragma unroll EPI_UNROLL
        for (int k = 0; k < READS; ++k) {
          const int qi = 64 * k + l;  // chunk index in the pass: row qi / CPR, chunk qi % CPR
          const int r = qi / CPR, ch = qi % CPR;
          const u32x4 d = *(const u32x4*)(stg + r * PITCH + (POW2 ? (((ch ^ r) & (CPR - 1)) << 4) : ch * 16));
          const int64_t row = wrow0 + pass * RP + r;
          // Non-temporal: the output bypasses the caches, so a tile's stores drain
          // faster and no dirty lines are left for the kernels that follow to write
          // back. Split partials too: re-read once by the reduction, they cost that
          // reduction a little but left dirty they slowed the casts that follow more
          // (MoE step 1.42-1.45 -> 1.36-1.38 ms, against plain stores on one device).
          if (row < row_limit)
            __builtin_nontemporal_store(d, (u32x4*)(T.out_base + ((row + row_shift) * p.ldo + wcol0) * ES + ch * 16));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int64_t row = wrow0 + 32 * i + (l & 31);
        if (row >= row_limit) continue;
        uint8_t* dst_row = T.out_base + ((row + row_shift) * p.ldo + wcol0 + 4 * h) * ES;
        const int cols_left = (int)(p.N - wcol0 - 4 * h);  // valid columns from this lane's first
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int c = 32 * j + 8 * q + e;
              if (c < cols_left) {
                if (OUT_BF16)
                  *(uint16_t*)(dst_row + c * 2) = (uint16_t)bf16x2_rne(acc[i][j][4 * q + e], 0.f);
                else
                  *(float*)(dst_row + c * 4) = acc[i][j][4 * q + e];
              }
            }
      }
    }
  };

  // ---- main loop -------------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = (v16f){};
  auto main_loop = [&](auto masked) {
    if (n_iter <= 0) return;
    for (int s = 0; s < NST - 1; ++s) issue_stage(s, s & 3, s < n_iter);
    wait_n(loads_after(0, NST - 2));
    __builtin_amdgcn_s_barrier();
#ifdef MX_CYCLE_STAMPS
    st_t1 = __builtin_amdgcn_s_memtime();
#endif
    // The main loop is unrolled by four (one 256-wide scale window), so window
    // boundaries, and the ring slots of a 2- or 4-deep ring, are compile-time
    // constants, and alternates two register sets, so no fragment is ever copied.
    Frag f0, f1;
    read_frags(f0, 0, k_first, masked);
    int64_t it = 0;
    for (; it + 4 <= n_iter; it += 4) {
      step(it, 0, f0, f1, masked);
      step(it + 1, 1, f1, f0, masked);
      step(it + 2, 2, f0, f1, masked);
      step(it + 3, 3, f1, f0, masked);
    }
    for (; it < n_iter; ++it) {  // 0 to 3 remaining steps
      step(it, (int)(it & 3), f0, f1, masked);
      f0 = f1;
    }
    MX_WAIT_VMCNT(0);  // every load has landed
    __builtin_amdgcn_s_barrier();  // every wave is done with the ring
#ifdef MX_CYCLE_STAMPS
    st_t2 = __builtin_amdgcn_s_memtime();
#endif
  };
  // bf16 K-grouped tiles whose range cuts a 16-byte chunk take the masked copy of
  // the loop; every other tile runs the loop without the per-step edge test (a
  // branch inside the step would split the MFMA / LDS-read interleaving)
  if constexpr (!SCALED && MODE == MODE_KGROUP) {
    if ((kb32 | ke32) & 15) main_loop(std::true_type{});
    else main_loop(std::false_type{});
  } else {
    main_loop(std::false_type{});
  }
  epilogue();
#ifdef MX_CYCLE_STAMPS
  const unsigned long long st_t3 = __builtin_amdgcn_s_memtime();
  const int64_t st_idx = (int64_t)blockIdx.x + (p.tail == TAIL_SUB ? kStampBlocks / 2 : 0);
  if (tid == 0 && st_idx < kStampBlocks) {
    const unsigned hw = __builtin_amdgcn_s_getreg(4 | (31 << 11));    // HW_ID: wave, SIMD, CU, SH, SE
    const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (31 << 11));  // XCC_ID
    unsigned long long* o = g_cycle_stamps + st_idx * 8;
    o[0] = st_t0; o[1] = st_t1; o[2] = st_t2; o[3] = st_t3; o[4] = st_rt;
    o[5] = ((unsigned long long)xcc << 32) | hw;
    o[6] = (unsigned long long)n_iter;
    o[7] = 1;
  }
#endif
}

}  // namespace mx

namespace {

constexpr int64_t kComputeUnits = 256;

// Launches one tile configuration and output type over the whole problem (p.splits
// already set), one block per tile or `grid` blocks.
template <int BM, int BN, int WGM, int WGN, int NST, int WPE, int MODE, int EL, int OUT_BF16>
hipError_t launch_cfg(mx::GemmArgs p, hipStream_t stream, int64_t grid = 0) {
  using C = mx::Cfg<BM, BN, WGM, WGN, NST>;
  const int64_t mt_extra = (MODE == mx::MODE_MGROUP && p.offs) ? p.groups : 0;
  p.mt_total = (p.M + BM - 1) / BM + mt_extra;
  p.nt = (p.N + BN - 1) / BN;
  p.tiles = MODE == mx::MODE_MGROUP ? p.mt_total * p.nt : (int64_t)p.splits * p.groups * p.mt_total * p.nt;
  if (p.tiles == 0) return hipSuccess;
  const int64_t blocks = grid > 0 ? grid : p.tiles;
  // the dynamic LDS limit of this instance, raised once per process (thread-safe
  // static initialisation)
  static const hipError_t attr = hipFuncSetAttribute((const void*)mx::k_gemm<BM, BN, WGM, WGN, NST, WPE, MODE, OUT_BF16, EL>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((mx::k_gemm<BM, BN, WGM, WGN, NST, WPE, MODE, OUT_BF16, EL>), dim3((unsigned)blocks),
                     dim3(C::THREADS), (size_t)C::LDS_BYTES, stream, p);
  return hipGetLastError();
}

// Sums the fp32 partials of `splits` contraction splits (split s at ws + s * stride)
// in split order into n outputs, fp32 or bf16. Four elements per thread.
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ ws, int splits, int64_t stride,
                                                      int64_t n, void* __restrict__ out, int out_bf16) {
  const int64_t step = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += step) {
    if (i + 4 <= n) {
      mx::v4f acc = *(const mx::v4f*)(ws + i);
      for (int s = 1; s < splits; ++s) acc += *(const mx::v4f*)(ws + s * stride + i);
      if (out_bf16)
        *(mx::u32x2*)((uint16_t*)out + i) = (mx::u32x2){mx::bf16x2_rne(acc[0], acc[1]), mx::bf16x2_rne(acc[2], acc[3])};
      else
        *(mx::v4f*)((float*)out + i) = acc;
    } else {
      for (int64_t j = i; j < n; ++j) {
        float a = ws[j];
        for (int s = 1; s < splits; ++s) a += ws[s * stride + j];
        if (out_bf16)
          ((uint16_t*)out)[j] = (uint16_t)mx::bf16x2_rne(a, 0.f);
        else
          ((float*)out)[j] = a;
      }
    }
  }
}

// K-grouped outputs with fewer 256x256 tiles than compute units, over a long
// contraction (weight gradients of narrow layers): split each group's contraction
// so the splits fill about one round of the chip. Returns 1 for no split.
int choose_splits(const mx::GemmArgs& p, int64_t elem_bytes) {
  const int64_t tiles = (int64_t)p.groups * ((p.M + 255) / 256) * ((p.N + 255) / 256);
  // half a round or more: 128x256 tiles fill the device without partials (a 4096 x
  // 2048 output over 4096 tokens: 44 us against 61 us split two ways)
  if (tiles >= kComputeUnits / 2 || tiles == 0) return 1;
  const int64_t wins_per_group = (p.K * elem_bytes + 255) / 256 / p.groups;  // 256-byte windows per group, on average
  int64_t s = kComputeUnits / tiles;
  s = std::min<int64_t>(s, wins_per_group / 2);  // at least two windows (8 k-steps) per split
  s = std::min<int64_t>(s, 16);
  return s >= 2 ? (int)s : 1;
}

// Tile configurations (block tile, wave grid, ring depth, blocks per compute unit):
enum Tiling {
  TILE_256 = 0,      // 256x256, 2x2 waves of 128x128, 4-deep ring, 136 KB LDS: one block per CU (M-grouped, bf16 out)
  TILE_128 = 1,      // 128x128, 2x2 waves of 64x64, 4-deep ring, 68 KB: two blocks per CU
  TILE_128x256 = 2,  // 128x256, 2x2 waves of 64x128, 3-deep ring, 80 KB: two blocks per CU
  TILE_192x256 = 3,  // 192x256, 1x4 waves of 192x64, 4-deep ring, 120 KB: one block per CU
  TILE_256_8W = 4,   // 256x256, 2x4 waves of 128x64, 4-deep ring, 144 KB: one block, two waves per SIMD
  TILE_256x192 = 5,  // 256x192, 2x2 waves of 128x96, 4-deep ring, 120 KB: one block per CU
};

template <int MODE, int EL, int OUT>
hipError_t launch_tiling_out(int tiling, const mx::GemmArgs& p, hipStream_t stream) {
  switch (tiling) {
    case TILE_128: return launch_cfg<128, 128, 2, 2, 4, 2, MODE, EL, OUT>(p, stream);
    case TILE_128x256: return launch_cfg<128, 256, 2, 2, 3, 2, MODE, EL, OUT>(p, stream);
    case TILE_192x256: return launch_cfg<192, 256, 1, 4, 4, 1, MODE, EL, OUT>(p, stream);
    case TILE_256_8W: return launch_cfg<256, 256, 2, 4, 4, 2, MODE, EL, OUT>(p, stream);
    case TILE_256x192: return launch_cfg<256, 192, 2, 2, 4, 1, MODE, EL, OUT>(p, stream);
    case TILE_256:
      // one wave per SIMD holds 256 fp32 accumulators: M-grouped bf16 output only (the
      // fp32 epilogue would spill; choose_tiling gives K-grouped tiles two waves per SIMD)
      if (OUT && MODE == mx::MODE_MGROUP) return launch_cfg<256, 256, 2, 2, 4, 1, MODE, EL, 1>(p, stream);
      return launch_cfg<256, 256, 2, 4, 4, 2, MODE, EL, OUT>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE, int EL>
hipError_t launch_tiling(int tiling, const mx::GemmArgs& p, int out_bf16, hipStream_t stream) {
  return out_bf16 ? launch_tiling_out<MODE, EL, 1>(tiling, p, stream) : launch_tiling_out<MODE, EL, 0>(tiling, p, stream);
}

// The tiling for a problem (p.splits set). Measured on the MoE training step's
// GEMMs (G=8, M=16384, K=N=4096, and a dense 576-wide layer), A/B inside the step on
// one device; every tiling gives bit-identical results, since each output element sums
// its k-steps in the same order.
template <int MODE, int EL>
int choose_tiling(const mx::GemmArgs& p, int out_bf16) {
  const int64_t groups_tiles = MODE == mx::MODE_KGROUP ? (int64_t)p.groups * p.splits : 1;
  const int64_t big_tiles = groups_tiles * ((p.M + 255) / 256) * ((p.N + 255) / 256);
  // few output tiles: quarter-size tiles spread the work over more compute units
  if (big_tiles < 128) return TILE_128;
  // a short contraction (a few k-steps per tile): the output stores dominate, and two
  // blocks per compute unit overlap one block's stores with the other's loop
  // (16384x4096 output over K=576: 55 us against 69-75 us for 256x256 tiles)
  if (MODE == mx::MODE_MGROUP && p.K <= 1024) return TILE_128x256;
  // M-grouped output columns that 192-column tiles cover with at least 1/8 less
  // padding than 256-column ones, in 128 or more tiles (the 576-wide forward: 576
  // against 768 columns, 44.5 against 48.3 us with eight-wave 256x256 tiles)
  if (MODE == mx::MODE_MGROUP && (p.N + 191) / 192 * 192 * 8 <= (p.N + 255) / 256 * 256 * 7 &&
      ((p.M + 255) / 256) * ((p.N + 191) / 192) >= 128)
    return TILE_256x192;
  // K-grouped output rows that 192-row tiles cover with at least 1/8 less padding
  // than 256-row ones (576 rows: 576 against 768, 58-59 us against 68-72 us); a
  // smaller saving does not repay the lower operand reuse of 192-row tiles (4096 rows
  // ran 294 us against 263 us as 256x256)
  if (MODE == mx::MODE_KGROUP && (p.M + 191) / 192 * 192 * 8 <= (p.M + 255) / 256 * 256 * 7) return TILE_192x256;
  // half a round to one round of 256x256 tiles: 128x256 tiles fill the device once
  // (the 4096 x 4096 x 2048 linear's dgrad, 128 tiles: 44 against 52 us; its wgrad
  // 44 against 61 us with the contraction split two ways)
  if (big_tiles < kComputeUnits) return TILE_128x256;
  // many tiles, bf16 output, M-grouped: one wave per SIMD (grouped forward / dgrad
  // 279-281 / 269-272 us against 287-288 / 277-278 with two). K-grouped wgrads take two
  // waves per SIMD: the bf16 one hides its masked, longer steps better (540 against
  // 564 us), and since the MFMAs split 3:1 around the k-step's wait the MXFP8 ones run
  // faster so too (inside the steps: MoE 286-287 against 290-291 us, 32-expert share
  // gate/up 1277 against 1296 us, down 611-612 against 633-636 us). fp32 output keeps
  // two waves per SIMD: 128 accumulators per wave leave room for the fp32 epilogue,
  // which with 256 spills (forward 286 against 287 us, wgrad 292 against 310 us)
  if (big_tiles >= 512 && out_bf16 && MODE == mx::MODE_MGROUP) return TILE_256;
  // otherwise (128-511 tiles: one round or two) two waves per SIMD hide each tile's
  // prologue and epilogue better (the 576-wide forward's single round of 192 tiles:
  // 53-54 us against 63-68 us)
  return TILE_256_8W;
}

// fp32 workspace bytes a K-grouped GEMM uses to split its contraction (0: no split).
int64_t split_workspace_bytes(const mx::GemmArgs& p, int64_t elem_bytes, int* splits_out, int64_t* stride_out) {
  const int splits = choose_splits(p, elem_bytes);
  const int64_t n_out = (int64_t)p.groups * p.M * p.N;
  const int64_t stride = (n_out + 3) / 4 * 4;  // keeps every partial 16-byte aligned
  if (splits_out) *splits_out = splits;
  if (stride_out) *stride_out = stride;
  return splits > 1 ? stride * splits * (int64_t)sizeof(float) : 0;
}

// K-grouped: with a caller workspace of at least split_workspace_bytes, narrow outputs
// split their contraction into fp32 partials that k_split_reduce sums in split order
// (deterministic); with less (or none) the contraction runs unsplit.
template <int MODE, int EL>
hipError_t launch(mx::GemmArgs& p, int out_bf16, void* ws, int64_t ws_bytes, hipStream_t stream) {
  p.splits = 1;
  if (MODE == mx::MODE_KGROUP) {
    int splits = 1;
    int64_t stride = 0;
    const int64_t need = split_workspace_bytes(p, EL == mx::EL_BF16 ? 2 : 1, &splits, &stride);
    if (need > 0 && ws && ws_bytes >= need) {
      const int64_t n_out = (int64_t)p.groups * p.M * p.N;
      mx::GemmArgs q = p;
      q.splits = splits;
      q.split_stride = stride;
      q.out = ws;
      hipError_t e = launch_tiling<MODE, EL>(choose_tiling<MODE, EL>(q, 0), q, 0, stream);
      if (e != hipSuccess) return e;
      const int64_t blocks = std::min<int64_t>((n_out + 1023) / 1024, 4096);
      hipLaunchKernelGGL(k_split_reduce, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, stream,
                         (const float*)ws, splits, stride, n_out, p.out, out_bf16);
      return hipGetLastError();
    }
  }
  const int tiling = choose_tiling<MODE, EL>(p, out_bf16);
  if (MODE == mx::MODE_MGROUP && p.offs && tiling == TILE_256 && out_bf16) {
    // whole rounds of 256x256 tiles, then the quarters of a short last round (the
    // MoE step's 1088 tiles: four rounds and 8 tiles per XCD as 256 quarters; inside
    // the step fwd 272 -> 263 us, dgrad 271-272 -> 265 us); when the device finds no
    // such round the second launch's blocks exit at once
    mx::GemmArgs main = p;
    main.tail = mx::TAIL_MAIN;
    hipError_t e = launch_tiling<MODE, EL>(tiling, main, out_bf16, stream);
    if (e != hipSuccess) return e;
    mx::GemmArgs rest = p;
    rest.tail = mx::TAIL_SUB;
    return launch_cfg<128, 128, 2, 2, 4, 2, MODE, EL, 1>(rest, stream, 2 * kComputeUnits);
  }
  return launch_tiling<MODE, EL>(tiling, p, out_bf16, stream);
}
}  // namespace

// M-grouped: C[m x n] = A[m x k] . B_g[n x k]^T per row group (forward and dgrad).
hipError_t mx_launch_gemm_mgroup(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                                 const int32_t* offs, const int32_t* offs_out, int groups, int64_t m, int64_t out_rows,
                                 int64_t n, int64_t k, void* out, int out_bf16, hipStream_t stream) {
  mx::GemmArgs p{};
  p.a = a; p.a_s = a_s; p.b = b; p.b_s = b_s; p.offs = offs; p.offs_out = offs_out; p.out = out;
  p.lda = k; p.ldb = k;
  p.a_rows = m; p.b_rows = (int64_t)groups * n;
  p.a_ktiles = p.b_ktiles = mx::scale_tiles_k(k / 32);
  p.M = m; p.N = n; p.K = k; p.ldo = n;
  p.out_rows = offs_out ? out_rows : m;
  p.groups = groups;
  return launch<mx::MODE_MGROUP, mx::EL_MXFP8>(p, out_bf16, nullptr, 0, stream);
}

// K-grouped: C_g[m x n] = A[m x K_g] . B[n x K_g]^T over each group's contraction range (wgrad).
hipError_t mx_launch_gemm_kgroup(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                                 const int32_t* offs, int groups, int64_t m, int64_t n, int64_t k, void* out,
                                 int out_bf16, void* ws, int64_t ws_bytes, hipStream_t stream) {
  mx::GemmArgs p{};
  p.a = a; p.a_s = a_s; p.b = b; p.b_s = b_s; p.offs = offs; p.out = out;
  p.lda = k; p.ldb = k;
  p.a_rows = m; p.b_rows = n;
  p.a_ktiles = p.b_ktiles = mx::scale_tiles_k(k / 32);
  p.M = m; p.N = n; p.K = k; p.ldo = n;
  p.groups = groups;
  return launch<mx::MODE_KGROUP, mx::EL_MXFP8>(p, out_bf16, ws, ws_bytes, stream);
}

// bf16 operands, no scales: the same two cores with pitches of 2 bytes per element.
hipError_t mx_launch_gemm_bf16_mgroup(const uint16_t* a, const uint16_t* b, const int32_t* offs, int groups,
                                      int64_t m, int64_t n, int64_t k, void* out, int out_bf16,
                                      hipStream_t stream) {
  mx::GemmArgs p{};
  p.a = (const uint8_t*)a; p.b = (const uint8_t*)b; p.offs = offs; p.out = out;
  p.lda = 2 * k; p.ldb = 2 * k;
  p.a_rows = m; p.b_rows = (int64_t)groups * n;
  p.M = m; p.N = n; p.K = k; p.ldo = n;
  p.out_rows = m;
  p.groups = groups;
  return launch<mx::MODE_MGROUP, mx::EL_BF16>(p, out_bf16, nullptr, 0, stream);
}

hipError_t mx_launch_gemm_bf16_kgroup(const uint16_t* a, const uint16_t* b, const int32_t* offs, int groups,
                                      int64_t m, int64_t n, int64_t k, void* out, int out_bf16, void* ws,
                                      int64_t ws_bytes, hipStream_t stream) {
  mx::GemmArgs p{};
  p.a = (const uint8_t*)a; p.b = (const uint8_t*)b; p.offs = offs; p.out = out;
  p.lda = 2 * k; p.ldb = 2 * k;
  p.a_rows = m; p.b_rows = n;
  p.M = m; p.N = n; p.K = k; p.ldo = n;
  p.groups = groups;
  return launch<mx::MODE_KGROUP, mx::EL_BF16>(p, out_bf16, ws, ws_bytes, stream);
}

// Scratch of mx_grouped_mm_wgrad_noalloc, for callers that cannot allocate: the
// split partials live here instead of in a caller workspace. One copy per device,
// held until the process ends; host code uses the address hipGetSymbolAddress gives
// for the current device (the array's name is only a host-side stand-in). Every split
// kernel writes all of its partial tiles, so nothing needs clearing between calls.
// Size: a split fills at most one round of kComputeUnits output tiles of 256 x 256
// fp32 partials (splits x tiles <= kComputeUnits), 64 MiB, so every call fits.
constexpr int64_t kNoAllocScratchBytes = kComputeUnits * 256 * 256 * (int64_t)sizeof(float);
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

int64_t mx_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// Device address of `scratch` on the current device, looked up once per device.
hipError_t mx_noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// Workspace bytes of a K-grouped call (dw [groups x n x k] over a contraction of m):
// what it needs to split its contraction, 0 if it does not split.
int64_t mx_kgroup_workspace_bytes(int groups, int64_t m, int64_t n, int64_t k, int bf16_operands) {
  mx::GemmArgs p{};
  p.groups = groups;
  p.M = n;
  p.N = k;
  p.K = m;
  return split_workspace_bytes(p, bf16_operands ? 2 : 1, nullptr, nullptr);
}

#ifdef MX_CYCLE_STAMPS
// Instrumented build only: copy out / clear the per-block records (8 x uint64 each,
// kStampBlocks blocks). Synchronous; for profiling runs, one call at a time.
extern "C" int64_t mx_cycle_stamps_blocks() { return mx::kStampBlocks; }
extern "C" int mx_cycle_stamps_read(void* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(mx::g_cycle_stamps), sizeof(mx::g_cycle_stamps), 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" int mx_cycle_stamps_clear() {
  static unsigned long long zeros[mx::kStampBlocks * 8];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(mx::g_cycle_stamps), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice);
}
#endif
