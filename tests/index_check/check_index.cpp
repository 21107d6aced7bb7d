// Host walk of the launches' index arithmetic (sparse_attention_chunk_amd/
// csrc/fm_index.h, the functions the kernels call), built by
// tests/test_index_bounds.py with g++, bounds-checked containers (.at()) and
// the address and undefined-behaviour sanitizers.  No GPU code runs here.
//
// Checked, over full, ragged, empty and long rows and several grid sizes:
//   - score grid: every valid chunk of every row belongs to exactly one
//     pipeline run, runs start on a tile, stay below the row's valid count
//     and within the record and score buffers, and are at most
//     kMaxSegTiles tiles long; the ragged plan's row of each wave's first
//     tile is the row holding that tile;
//   - threshold-fused pass: the mask words of the runs of a row are
//     disjoint, inside the row, and cover every valid chunk below the row's
//     last whole word;
//   - top-K scan and finish: every tile word the scan writes is inside its
//     row of tile_info_stride(N) words, each tile the finish reads is written
//     exactly once, and the tile size leaves at least 4 K tiles when it is
//     larger than 16.
// Prints "checked ..." and exits 0, or names the shape and the failed check
// and exits 1.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fm_index.h"

using namespace fm::idx;

namespace {

constexpr int64_t kRecordBytes = 132;  // one chunk's record
constexpr int kScanThreads = 256;      // top-K scan block

const char* g_shape = "";

#define CHECK(cond)                                                                        \
  do {                                                                                     \
    if (!(cond)) {                                                                         \
      std::fprintf(stderr, "FAIL %s (line %d) for %s\n", #cond, __LINE__, g_shape);        \
      std::exit(1);                                                                        \
    }                                                                                      \
  } while (0)

struct Shape {
  int B;
  int64_t N;
  std::vector<int32_t> valid;  // empty: full rows
};

int64_t g_runs = 0, g_shapes = 0, g_scans = 0;

void check_score_walk(const Shape& sh, int waves) {
  const int B = sh.B;
  const int64_t N = sh.N;
  const bool ragged = !sh.valid.empty();
  const int32_t* vptr = ragged ? sh.valid.data() : nullptr;
  // The ragged plan's outputs (the ragged launch's plan block forms the same prefix with a
  // parallel scan): each row's first list index and each wave's first row.
  std::vector<int64_t> pre(B + 1);
  std::vector<int32_t> wave_row(waves);
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    pre.at(b) = total;
    total += row_tile_count(clamp_valid(vptr, b, N));
  }
  pre.at(B) = total;
  if (ragged)
    for (int g = 0; g < waves; ++g) {
      int64_t first, end;
      wave_share(g, waves, total, &first, &end);
      const int r = plan_row_of(pre.data(), B, first);
      CHECK(r >= 0 && r < B);
      // The row holding list index `first` (when the share is not empty).
      if (first < end) CHECK(pre.at(r) <= first && first < pre.at(r + 1));
      wave_row.at(g) = r;
    }
  const int64_t total_tiles = (int64_t)B * row_tile_count(N);
  std::vector<std::vector<uint8_t>> cover(B, std::vector<uint8_t>(N, 0));
  std::vector<std::vector<uint8_t>> words(B, std::vector<uint8_t>(N, 0));
  for (int g = 0; g < waves; ++g) {
    walk_runs(g, waves, B, N, vptr, ragged ? pre.data() : nullptr, ragged ? wave_row.data() : nullptr, total_tiles,
              [&](int b, int64_t start, int64_t count) {
                ++g_runs;
                CHECK(b >= 0 && b < B);
                const int64_t vn = clamp_valid(vptr, b, N);
                CHECK(start >= 0 && start % kTile == 0);
                CHECK(count > 0 && start + count <= vn);
                CHECK(count <= kMaxSegTiles * kTile);
                // Records [(b N + start) 132, + count 132) and scores
                // [b N + start, + count) inside their [B][N] buffers, with
                // the run's byte counts in 32 bits.
                CHECK(((int64_t)b * N + start + count) * kRecordBytes <= (int64_t)B * N * kRecordBytes);
                CHECK(count * kRecordBytes < ((int64_t)1 << 31));
                for (int64_t n = start; n < start + count; ++n) cover.at(b).at(n)++;
                const int64_t w = run_mask_words(start, count, N);
                CHECK(w >= 0 && w % 4 == 0 && start + w <= N);
                for (int64_t n = start; n < start + w; ++n) words.at(b).at(n)++;
              });
  }
  for (int b = 0; b < B; ++b) {
    const int64_t vn = clamp_valid(vptr, b, N);
    const int64_t whole = N & ~(int64_t)3;
    for (int64_t n = 0; n < N; ++n) {
      CHECK(cover.at(b).at(n) == (n < vn ? 1 : 0));
      CHECK(words.at(b).at(n) <= 1);
      if (n < vn && n < whole) CHECK(words.at(b).at(n) == 1);
    }
  }
}

void check_topk_scan(const Shape& sh, int32_t k) {
  const int B = sh.B;
  const int64_t N = sh.N;
  const int32_t* vptr = sh.valid.empty() ? nullptr : sh.valid.data();
  const int64_t stride = tile_info_stride(N);
  const int64_t slice = (int64_t)kScanThreads * kSelSub;
  const int64_t slices = (N + slice - 1) / slice;
  for (int b = 0; b < B; ++b) {
    const int64_t vn = clamp_valid(vptr, b, N);
    if (k <= 0 || (int64_t)k >= vn) continue;  // the scan writes the mask alone
    ++g_scans;
    const int s = tile_shift(vn, k);
    CHECK(s >= 0 && s <= 2);
    const int64_t nt = finish_tiles(vn, s);
    CHECK(nt >= 1 && nt <= stride);
    if (s > 0) CHECK(nt >= 4 * (int64_t)k);
    std::vector<uint8_t> written(stride, 0);
    for (int64_t blk = 0; blk < slices; ++blk) {
      if (blk * slice >= vn) continue;  // blocks past vn write no tile word
      for (int t = 0; t < kScanThreads; ++t) {
        const int64_t g = blk * kScanThreads + t;
        const int64_t tile = scan_tile_written(g, s, vn);
        if (tile < 0) continue;
        CHECK(tile < stride);
        written.at(tile)++;
      }
    }
    for (int64_t t = 0; t < stride; ++t) CHECK(written.at(t) == (t < nt ? 1 : 0));
  }
}

uint64_t g_rng = 0x9e3779b97f4a7c15ull;
uint64_t next_rand() {  // xorshift64*
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return g_rng * 0x2545f4914f6cdd1dull;
}

void run_shape(const Shape& sh, const char* name, std::initializer_list<int> waves) {
  char buf[256];
  std::snprintf(buf, sizeof buf, "%s (B=%d N=%" PRId64 ")", name, sh.B, sh.N);
  g_shape = buf;
  ++g_shapes;
  for (int w : waves) check_score_walk(sh, w);
  for (int32_t k : {1, 3, 64, 512, 1024, 4096}) check_topk_scan(sh, k);
  if (!sh.valid.empty())
    for (int b = 0; b < sh.B; ++b) {
      const int64_t vn = clamp_valid(sh.valid.data(), b, sh.N);
      for (int64_t k : {vn - 1, vn, vn + 1})
        if (k > 0 && k < (int64_t)1 << 30) check_topk_scan(sh, (int32_t)k);
    }
}

}  // namespace

int main() {
  const int64_t Ns[] = {1, 15, 16, 17, 63, 100, 1024, 4095, 4096, 4097, 12289, 65539};
  for (int B : {1, 2, 3, 30}) {
    for (int64_t N : Ns) {
      run_shape(Shape{B, N, {}}, "full rows", {4, 28, 1024, 4096});
      Shape r{B, N, std::vector<int32_t>(B)};
      for (int b = 0; b < B; ++b) {
        const uint64_t x = next_rand();
        switch (x % 6) {
          case 0: r.valid[b] = 0; break;
          case 1: r.valid[b] = (int32_t)N; break;
          case 2: r.valid[b] = (int32_t)(N + 1 + (x >> 8) % 100); break;  // clamped to N
          case 3: r.valid[b] = -(int32_t)((x >> 8) % 7) - 1; break;      // clamped to 0
          default: r.valid[b] = (int32_t)((x >> 8) % (uint64_t)(N + 1)); break;
        }
      }
      run_shape(r, "ragged rows", {4, 28, 1024, 4096});
      Shape z{B, N, std::vector<int32_t>(B, 0)};
      run_shape(z, "empty rows", {4, 1024});
    }
  }
  // The workloads' shapes: 30 x 262144 full, 60 x 131072 ragged, 64 x 8192.
  run_shape(Shape{30, 262144, {}}, "b30 n262144", {1024});
  {
    Shape r{60, 131072, std::vector<int32_t>(60)};
    for (int b = 0; b < 60; ++b) r.valid[b] = (int32_t)(next_rand() % 131073);
    run_shape(r, "b60 n131072 ragged", {1024});
  }
  run_shape(Shape{64, 8192, {}}, "b64 n8192", {1024, 4096});
  // Shares longer than kMaxSegTiles tiles (split into several runs).
  run_shape(Shape{1, (int64_t)1 << 22, {}}, "long row", {2, 4});
  {
    Shape r{2, (int64_t)1 << 21, {(int32_t)((1 << 21) - 5), 7}};
    run_shape(r, "long ragged rows", {1, 3});
  }
  std::printf("checked %" PRId64 " shapes, %" PRId64 " pipeline runs, %" PRId64 " top-K rows\n", g_shapes, g_runs,
              g_scans);
  return 0;
}
