// Index arithmetic of the launches, shared by the kernels and a host-side
// bounds checker: plain C++ with no HIP types or builtins, so the functions
// the kernels run also compile on the host, where tests/index_check walks
// them over many shapes with bounds-checked containers and the address and
// undefined-behaviour sanitizers.
//
// Covered: the score grid's split of the tile list into wave shares and
// pipeline runs (full and ragged rows), the ragged plan's row of each
// wave's first tile, the threshold mask words a run writes, and the top-K
// scan's tile size and tile-word rows.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define FM_HD __host__ __device__
#else
#define FM_HD
#endif

namespace fm {
namespace idx {

constexpr int kTile = 16;                     // chunks per score tile (one MFMA column tile)
constexpr int64_t kMaxSegTiles = 1 << 16;     // tiles per pipeline run
constexpr int kSelSub = 16;                   // chunks per top-K scan thread

// A row's valid chunks: valid_n clamped to [0, N] (N without valid_n).
FM_HD inline int64_t clamp_valid(const int32_t* valid_n, int b, int64_t N) {
  if (!valid_n) return N;
  const int64_t v = valid_n[b];
  return v < 0 ? 0 : (v > N ? N : v);
}

// Tiles of a row of vn valid chunks.
FM_HD inline int64_t row_tile_count(int64_t vn) { return (vn + kTile - 1) / kTile; }

// Wave gw's share [*t, *t_end) of a list of `total` tiles split over
// `waves` waves: contiguous, in order, sizes differing by at most one.
FM_HD inline void wave_share(int64_t gw, int64_t waves, int64_t total, int64_t* t, int64_t* t_end) {
  *t = gw * total / waves;
  *t_end = (gw + 1) * total / waves;
}

// The ragged plan's row of the tile at list index `first`: the largest row
// b with pre[b] <= first, pre holding each row's first list index (pre[0]
// = 0, non-decreasing, B entries).
FM_HD inline int plan_row_of(const int64_t* pre, int B, int64_t first) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= first) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The pipeline runs of wave gw's share: the valid tiles of all rows, in
// row-major order, cut into equal contiguous shares (wave_share).  With
// row_tiles (prefix of the rows' valid tile counts, B + 1 entries) and
// wave_row (row of each wave's first tile) the rows are ragged; without,
// every row has ceil(N / 16) tiles and total_tiles is the list length.  A
// share may end in a later row: each row's part is its own run, at most
// kMaxSegTiles tiles long, run(b, start, count) with start a multiple of 16
// and start + count <= the row's valid chunks.
template <class Run>
FM_HD inline void walk_runs(int64_t gw, int64_t waves, int B, int64_t N, const int32_t* valid_n,
                            const int64_t* row_tiles, const int32_t* wave_row, int64_t total_tiles, Run&& run) {
  const int64_t total = row_tiles ? row_tiles[B] : total_tiles;
  int64_t t, t_end;
  wave_share(gw, waves, total, &t, &t_end);
  if (t >= t_end) return;
  const int64_t row_full = (N + kTile - 1) / kTile;
  int b;
  int64_t first;  // list index of row b's first tile
  if (row_tiles) {
    b = wave_row[gw];
    first = row_tiles[b];
  } else {
    b = (int)(t / row_full);
    first = (int64_t)b * row_full;
  }
  while (t < t_end) {
    const int64_t last = row_tiles ? row_tiles[b + 1] : first + row_full;
    int64_t run_end = t_end < last ? t_end : last;
    if (run_end - t > kMaxSegTiles) run_end = t + kMaxSegTiles;
    if (run_end > t) {
      const int64_t vn = clamp_valid(valid_n, b, N);
      const int64_t start = (t - first) * kTile;
      const int64_t end = run_end == last ? vn : (run_end - first) * kTile;
      run(b, start, end - start);
    }
    t = run_end;
    if (t >= last) {
      ++b;
      first = last;
    }
  }
}

// Mask bytes a run of the threshold-fused score pass writes, as whole
// 4-byte words from its first chunk: up to its last chunk rounded up to a
// word, but never past the row's last whole word (a run starts on a tile,
// so that word ends at N - N % 4 in every run of the row; the row's last
// N % 4 bytes are written by a separate kernel).
FM_HD inline int64_t run_mask_words(int64_t start, int64_t count, int64_t N) {
  const int64_t words = (count + 3) & ~(int64_t)3;
  const int64_t row_words = (N - start) & ~(int64_t)3;
  return words < row_words ? words : row_words;
}

// Top-K scan: log2 of the kSelSub-chunk parts per tile (0..2) in a row of
// vn chunks, the largest leaving at least 4 K tiles.
FM_HD inline int tile_shift(int64_t vn, int32_t k) {
  const int64_t need = 4 * (int64_t)k;
  return (vn >> 6) >= need ? 2 : ((vn >> 5) >= need ? 1 : 0);
}
// Tile words per row: ceil(N / 16) rounded up to a multiple of 2 (16-byte
// aligned rows), enough for the smallest tile.
FM_HD inline int64_t tile_info_stride(int64_t N) { return ((N + 15) / 16 + 1) & ~(int64_t)1; }
// The tile word scan thread g (of a row of vn chunks, shift s) writes, or
// -1: the first thread of each tile that starts below vn writes it.
FM_HD inline int64_t scan_tile_written(int64_t g, int s, int64_t vn) {
  const int64_t tile = g >> s;
  const bool first = (g & ((1 << s) - 1)) == 0;
  return first && (tile << (4 + s)) < vn ? tile : -1;
}
// Tiles of a row the top-K finish reads (tile words written by the scan).
FM_HD inline int64_t finish_tiles(int64_t vn, int s) { return (vn + (kSelSub << s) - 1) >> (4 + s); }
static_assert(kSelSub == 16, "finish_tiles shifts by log2(kSelSub) = 4");

}  // namespace idx
}  // namespace fm
