// Tile bookkeeping of the persistent grouped GEMM, written once for the device
// (the kernel's scheduler) and the host (a CPU bounds check of the same code).
//
// Group g (an expert) owns the rows [bound[g], bound[g+1]) of the A operand and
// of the output.  The bounds come from device memory that a caller fills (the
// row offsets of moe_grouped_ffn), so they are not trusted: each bound is the
// running maximum of the raw offsets up to it, clamped to [0, M].  Consistent
// offsets (non-decreasing, last <= M) pass through unchanged; anything else
// still gives segments that are disjoint, in order and inside [0, M), so no
// tile reads or writes a row outside the buffers.
//
// Inside a group the tiles run in chunks of m_chunk row tiles; inside a chunk,
// in column groups of n_group column tiles; inside a column group, row tile by
// row tile (tile_spot).
#pragma once

#include <stdint.h>

#ifndef MOE_HD
#define MOE_HD __host__ __device__
#endif

namespace moe {

// v clamped to [lo, hi] (lo <= hi)
MOE_HD inline int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

// The next segment bound: the running maximum of the raw offsets (prev_max is the
// maximum of the raw offsets before this one), clamped to [0, M].
MOE_HD inline int64_t segment_bound(int64_t prev_max, int64_t raw, int64_t M) {
  return clamp64(raw > prev_max ? raw : prev_max, 0, M);
}

// Tiles of a group with `rows` rows (rows >= 0), ntn column tiles each.
MOE_HD inline int64_t group_tiles(int64_t rows, int BM, int ntn) { return (rows + BM - 1) / BM * (int64_t)ntn; }

// A tile prefix entry, saturated so that it fits an int: groups whose first tile
// would lie past INT32_MAX own no tile.
MOE_HD inline int saturate_tiles(int64_t v) { return v > 0x7fffffffLL ? 0x7fffffff : (int)v; }

struct TileSpot {
  int mt, nt;   // row tile (within the group) and column tile
};

// Position of the group's local-th tile (0 <= local < mtc * ntn) for mtc row tiles
// and ntn column tiles, in chunks of m_chunk row tiles (<= 0: one chunk) and
// column groups of n_group column tiles (<= 0: one group).
MOE_HD inline TileSpot tile_spot(int local, int mtc, int ntn, int m_chunk, int n_group) {
  const int SM = (m_chunk > 0 && m_chunk < mtc) ? m_chunk : mtc;
  const int NG = (n_group > 0 && n_group < ntn) ? n_group : ntn;
  const int ch = local / (SM * ntn);
  const int base_m = ch * SM;
  const int sm = (mtc - base_m) < SM ? (mtc - base_m) : SM;
  const int l = local - ch * SM * ntn;
  const int cg = l / (sm * NG);
  const int l2 = l - cg * sm * NG;
  const int sz = (ntn - cg * NG) < NG ? (ntn - cg * NG) : NG;
  TileSpot s;
  s.mt = base_m + l2 / sz;
  s.nt = cg * NG + l2 % sz;
  return s;
}

// The group owning tile `tile` (0 <= tile < tstart[G]): the largest g with
// tstart[g] <= tile, where tstart[0..G] is the non-decreasing tile prefix.  Empty
// groups share their start with the next group, which this picks.
MOE_HD inline int find_group(const int* tstart, int G, int tile) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tstart[mid] <= tile) lo = mid; else hi = mid;
  }
  return lo;
}

// Source row of a gather map entry, clamped to the rows that exist ([0, n_rows)).
MOE_HD inline int32_t clamp_row(int32_t r, int64_t n_rows) {
  return r < 0 ? 0 : ((int64_t)r >= n_rows ? (int32_t)(n_rows - 1) : r);
}

}  // namespace moe
