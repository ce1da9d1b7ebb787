// CPU check of the grouped GEMM's tile bookkeeping (csrc/tile_walk.h, the same
// functions the kernel calls), composed the way the kernel composes them:
// segment bounds from raw device offsets, the saturating tile prefix, the group
// lookup and the tile position inside a group.  For every tile of every case it
// checks that the rows and columns the tile reads and writes lie inside the
// buffers (rows [0, M), gather rows [0, n_in), columns [0, N)), and, for
// consistent offsets, that every (group, row tile, column tile) is visited
// exactly once.  Cases: consistent ragged offsets (empty groups, a group past
// the 16-row-tile chunk with a short last chunk), and offsets that are negative,
// past M, decreasing or enormous.  Exit status 0 = every check passed.
#define MOE_HD
#include "tile_walk.h"

#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <tuple>
#include <vector>

using namespace moe;

static int failures = 0;
#define CHECK(c, ...)                              \
  do {                                             \
    if (!(c)) {                                    \
      if (failures < 20) {                         \
        std::printf("FAIL %s: ", #c);              \
        std::printf(__VA_ARGS__);                  \
        std::printf("\n");                         \
      }                                            \
      ++failures;                                  \
    }                                              \
  } while (0)

struct Case {
  const char* name;
  std::vector<int32_t> seg;   // G + 1 raw offsets
  int64_t M;                  // rows of the buffers (n_max)
  int BM, N, NOUT, m_chunk, n_group;
  bool consistent;
  int64_t tile_cap;           // only walk this many tiles (saturated prefixes)
};

static void run(const Case& c) {
  const int G = (int)c.seg.size() - 1;
  const int ntn = (c.N + c.NOUT - 1) / c.NOUT;
  // bounds: the running maximum of the raw offsets, clamped (build_tile_prefix)
  std::vector<int> bound(G + 1);
  int64_t run = INT64_MIN;
  for (int i = 0; i <= G; ++i) {
    bound[i] = (int)segment_bound(run, c.seg[i], c.M);
    run = run > c.seg[i] ? run : c.seg[i];
  }
  std::vector<int> tstart(G + 1);
  int64_t acc = 0;
  for (int g = 0; g < G; ++g) {
    CHECK(bound[g] <= bound[g + 1], "%s: bounds decrease at %d", c.name, g);
    CHECK(bound[g] >= 0 && bound[g + 1] <= c.M, "%s: bound outside [0, M] at %d", c.name, g);
    tstart[g] = saturate_tiles(acc);
    acc += group_tiles((int64_t)bound[g + 1] - bound[g], c.BM, ntn);
  }
  tstart[G] = saturate_tiles(acc);
  const int total = tstart[G];
  const int64_t walk = total < c.tile_cap ? total : c.tile_cap;
  std::set<std::tuple<int, int, int>> seen;
  std::mt19937 rng(7);
  for (int64_t i = 0; i < walk; ++i) {
    // saturated cases: the first and last tiles plus random ones
    const int tile = (walk == total) ? (int)i
                     : (i < walk / 2 ? (int)i : (int)(total - 1 - (int64_t)(rng() % (uint32_t)(total < 1000000 ? total : 1000000))));
    const int g = find_group(tstart.data(), G, tile);
    CHECK(g >= 0 && g < G, "%s: tile %d -> group %d", c.name, tile, g);
    const int local = tile - tstart[g];
    const int64_t lo = bound[g], hi = bound[g + 1];
    const int mtc = (int)((hi - lo + c.BM - 1) / c.BM);
    CHECK(local >= 0 && (int64_t)local < (int64_t)mtc * ntn, "%s: tile %d local %d of %d x %d", c.name, tile, local,
          mtc, ntn);
    const TileSpot sp = tile_spot(local, mtc, ntn, c.m_chunk, c.n_group);
    CHECK(sp.mt >= 0 && sp.mt < mtc && sp.nt >= 0 && sp.nt < ntn, "%s: spot (%d, %d) of (%d, %d)", c.name, sp.mt,
          sp.nt, mtc, ntn);
    const int64_t m0 = lo + (int64_t)sp.mt * c.BM;
    const int64_t rows_valid = (hi - m0) < c.BM ? (hi - m0) : c.BM;
    CHECK(rows_valid >= 1 && m0 >= 0 && m0 + rows_valid <= c.M, "%s: rows [%lld, %lld) outside [0, %lld)", c.name,
          (long long)m0, (long long)(m0 + rows_valid), (long long)c.M);
    CHECK(sp.nt * c.NOUT < c.N, "%s: column tile %d past N", c.name, sp.nt);
    if (c.consistent) {
      const bool fresh = seen.insert(std::make_tuple(g, sp.mt, sp.nt)).second;
      CHECK(fresh, "%s: tile (%d, %d, %d) visited twice", c.name, g, sp.mt, sp.nt);
    }
  }
  if (c.consistent) {
    int64_t want = 0;
    for (int g = 0; g < G; ++g) want += group_tiles((int64_t)c.seg[g + 1] - c.seg[g], c.BM, ntn);
    CHECK((int64_t)seen.size() == want, "%s: %zu tiles visited, %lld expected", c.name, seen.size(), (long long)want);
    for (int g = 0; g <= G; ++g) CHECK(bound[g] == c.seg[g], "%s: consistent offset %d changed", c.name, g);
  }
  std::printf("%-28s G=%d M=%lld tiles=%d walked=%lld\n", c.name, G, (long long)c.M, total, (long long)walk);
}

static std::vector<int32_t> offsets_of(const std::vector<int>& counts) {
  std::vector<int32_t> o(1, 0);
  for (int x : counts) o.push_back(o.back() + x);
  return o;
}

int main() {
  std::vector<Case> cases;
  // the forward's launch shapes: 256-row tiles, gate/up 128 output columns per
  // tile (F = 384 -> 3), down 256 (d = 768 -> 3); 16 x 2 chunks (8 x 2, the
  // forward's current order, below)
  auto fwd = [&](const char* n, std::vector<int> counts, int N, int NOUT) {
    const auto o = offsets_of(counts);
    cases.push_back({n, o, (int64_t)o.back() + 37, 256, N, NOUT, 16, 2, true, INT64_MAX});
  };
  fwd("ragged gate/up", {4400, 0, 300, 37}, 384, 128);
  fwd("ragged down", {4400, 0, 300, 37}, 768, 256);
  fwd("one long expert", {5000, 0, 3}, 192, 128);
  fwd("exact chunks", {8192, 4096, 0, 1}, 1792, 128);
  fwd("page shape skew", {27781, 226, 5000, 0, 4097, 4095, 4096}, 6144, 256);
  // the forward's chunks of 8 row tiles (the ones above use 16)
  auto fwd8 = [&](const char* n, std::vector<int> counts, int N, int NOUT) {
    const auto o = offsets_of(counts);
    cases.push_back({n, o, (int64_t)o.back() + 37, 256, N, NOUT, 8, 2, true, INT64_MAX});
  };
  fwd8("ragged gate/up, chunks of 8", {4400, 0, 300, 37}, 384, 128);
  fwd8("page shape skew, chunks of 8", {27781, 226, 5000, 0, 4097, 4095, 4096}, 1792, 128);
  fwd8("one long expert, chunks of 8", {5000, 0, 3}, 6144, 256);
  std::mt19937 rng(1);
  for (int r = 0; r < 20; ++r) {
    std::vector<int> counts(1 + rng() % 60);
    for (auto& x : counts) x = (rng() % 4 == 0) ? 0 : (int)(rng() % 9000);
    static char names[20][32];
    std::snprintf(names[r], 32, "random %d", r);
    fwd(names[r], counts, 64 * (1 + rng() % 40), (rng() % 2) ? 128 : 256);
  }
  // offsets a caller got wrong
  cases.push_back({"negative and past M", {-50, 100, 700, 100000, 90}, 1000, 256, 512, 128, 16, 2, false, INT64_MAX});
  cases.push_back({"decreasing", {900, 10, 500, 20, 1000}, 1000, 256, 512, 256, 16, 2, false, INT64_MAX});
  cases.push_back({"all past M", {5000, 6000, 7000}, 1000, 256, 256, 128, 16, 2, false, INT64_MAX});
  cases.push_back({"alternating full", {0, 2000000000, 0, 2000000000, 0, 2000000000}, 2000000000, 256, 6144, 128,
                   16, 2, false, 200000});
  {
    std::vector<int32_t> seg(1025);
    for (auto& v : seg) v = (int32_t)((int64_t)(rng() % 4000000000u) - 2000000000);
    cases.push_back({"random garbage 1024", seg, 2000000000, 256, 8192, 128, 16, 2, false, 200000});
  }
  for (const auto& c : cases) run(c);
  // gather rows: clamped into [0, n_in)
  const int32_t raw[] = {-7, 0, 5, 99, 100, 101, 2147483647, (int32_t)0x80000000};
  for (int32_t r : raw) {
    const int32_t q = clamp_row(r, 100);
    CHECK(q >= 0 && q < 100 && (r < 0 || r >= 100 || q == r), "clamp_row(%d, 100) = %d", r, q);
  }
  std::printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
