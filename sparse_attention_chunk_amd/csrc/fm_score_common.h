// Parts shared by the two score kernels (the f16-MFMA path in fm_score.hip
// and the fp8-MFMA path in fm_score_fp8.hip): record tiles and their loads,
// the per-lane buffer views of one pipeline run, the cross-lane head sum, the
// ensemble and store of a tile's scores (per tile, or per group of four
// tiles), the threshold mask, and the walk of a wave's share of the tile
// list.
//
// Both paths put the keys in the MFMA's B operand: lane l holds chunk l % 16
// of a 16-chunk tile and the 32 code bytes at dims 32 (l / 16) .. + 31, and
// receives the dot products of heads 4 (l / 16) + r (r = 0..3) of a 16-head
// tile with that chunk.
#pragma once

#include "fm_internal.h"

namespace fm {
namespace score {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kTile = idx::kTile;                // chunks per MFMA column tile
constexpr int kTileBytes = kTile * kRecord;      // 2112
constexpr int kRing = 8;                         // register ring of record tiles
constexpr int kAhead = 6;                        // tile i + 6 is requested in the phase of tile i
// A lane offset past every buffer of one pipeline run: the access is
// dropped by the range check, with no branch.
constexpr uint32_t kDropOffset = 0x40000000u;
// A run of at most idx::kMaxSegTiles tiles addresses tiles below
// kMaxSegTiles + 16 (the loop's rounding up to 8 m + 1 tiles, kAhead tiles
// requested ahead, the last group of four), so every tile offset (the
// scalar offset of a load or store) stays below 2^28: a run's buffers are
// smaller than kDropOffset, and kDropOffset plus a tile offset does not
// wrap around 2^32.
static_assert((idx::kMaxSegTiles + 16) * (int64_t)kTileBytes < (1 << 28), "tile offsets reach 2^28");

// Cross-lane moves.  permlane32_swap(x, y) swaps lanes 32..63 of x with
// lanes 0..31 of y; permlane16_swap(x, y) swaps the odd 16-lane rows of x
// with the even rows of y.  Both return the new (x, y).
__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Sum and max over the four 16-lane rows {l, l^16, l^32, l^48} (every lane
// gets it).
__device__ __forceinline__ float sum4rows(float v) {
  float w = v;
  swap32(v, w);
  v += w;
  w = v;
  swap16(v, w);
  return v + w;
}
// max(a, b) as the median of (a, b, pinf) with pinf = +inf held in a
// register the compiler cannot see into: one instruction.  (With a literal
// +inf the compiler rewrites the median as a maximum and quiets both
// operands first, two more instructions; the scores are never NaN.)
__device__ __forceinline__ float max2(float a, float b, float pinf) {
  return __builtin_amdgcn_fmed3f(a, b, pinf);
}
__device__ __forceinline__ float max4rows(float v, float pinf) {
  float w = v;
  swap32(v, w);
  v = max2(v, w, pinf);
  w = v;
  swap16(v, w);
  return max2(v, w, pinf);
}

// Sum (SUM) or maximum over the four 16-lane rows of four tiles at once:
// lane row g of the result holds the reduction of x_k with k = kGroupTile[g]
// (rows 1 and 2 trade places), each lane's column c staying chunk c.  Two
// 32-lane swaps pair rows {0, 2} and {1, 3} of x0 with x1 and of x2 with x3,
// one 16-lane swap then pairs the halves: 3 swaps and 3 operations for four
// tiles, where one tile alone takes 2 swaps, 2 moves and 2 operations.  The
// sums associate as sum4rows' do, (r0 + r2) + (r1 + r3).
template <bool SUM>
__device__ __forceinline__ float reduce4(float x0, float x1, float x2, float x3, float pinf) {
  swap32(x0, x1);
  swap32(x2, x3);
  float a = SUM ? x0 + x1 : max2(x0, x1, pinf);
  float b = SUM ? x2 + x3 : max2(x2, x3, pinf);
  swap16(a, b);
  return SUM ? a + b : max2(a, b, pinf);
}
constexpr int kGroupTile[4] = {0, 2, 1, 3};

// The three layers' logits of every chunk from the lanes' partial sums:
// u[l] is lane group g's part of layer l for the lane's chunk (l % 16).
// Layers 0 and 1 share the first swap (lanes 0..31 then hold layer 0's sums
// over the row pairs {r, r + 2}, lanes 32..63 layer 1's), layer 2 takes the
// other operand; the second swap completes the sums.  Returns, per 16-lane
// row, one layer's total: row 0 layer 0, row 1 layer 2, row 2 layer 1, and
// row 3 layer 2 again (dup_zero false) or 0 (dup_zero true).
__device__ __forceinline__ float layer_totals(const float (&u)[kLayers], bool dup_zero) {
  float a = u[0], b = u[1], c = u[2], d = dup_zero ? 0.f : u[2];
  swap32(a, b);
  swap32(c, d);
  float ab = a + b, cd = c + d;
  swap16(ab, cd);
  return ab + cd;
}
// 16-lane row of each layer's total in layer_totals' result.
constexpr int kLayerRow[kLayers] = {0, 2, 1};

__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

struct RawTile {
  u32x4 lo, hi;  // this lane's 32 code bytes
  float s;       // the chunk's scale
};

// One pipeline run's buffers: base addresses and byte counts of this
// run's records and outputs (wave-uniform), and the lane's offsets within a
// tile.  Record loads and group stores use one descriptor over the run with
// the tile's offset in the scalar offset; per-tile stores use a descriptor
// starting at the tile (tile_rsrc).  Either way the per-lane offsets stay
// fixed and the range checks make reads past the run return 0 and drop
// writes past it.
struct Ctx {
  const uint8_t* rec;                    // records of this run's chunks
  float* out;                            // their scores
  float* pl[kLayers];                    // their per-layer scores (when requested)
  int32_t rec_bytes, out_bytes;          // 132 and 4 bytes per chunk of the run
  uint32_t lane_rec_off;                 // 132 c + 32 g
  uint32_t lane_scale_off;               // 132 c + 128
  uint32_t lane_out_off;                 // 4 c in lane group 0, out of range elsewhere
  uint32_t lane_pl_off[kLayers];         // 4 c in the lane row holding layer l's total, out of range elsewhere
  int c, g;
  // Threshold mask folded into the pass (unused without it).
  uint8_t* mask;                         // mask bytes of this run's chunks
  int32_t count;                         // chunks in the run
  int32_t mask_words;                    // mask bytes written as whole words: the run's words inside its row
  uint32_t lane_mask_off;                // 4 l in lanes l = 0..3 (one word of 4 mask bytes each), out of range elsewhere
  uint32_t nib_shift;                    // 4 (l % 4): lane l's four chunks in the tile's compare mask
  float threshold;
  // Four-tile groups (scores only): lane l stores chunk c of tile
  // kGroupTile[g] of the group, i.e. group chunk 16 kGroupTile[g] + c; the
  // group's mask goes out as 16 words from lanes 0..15.
  uint32_t lane_grp_off;                 // 4 (16 kGroupTile[g] + c)
  int32_t grp_chunk;                     // 16 kGroupTile[g] + c
  uint32_t lane_grp_mask_off;            // 4 c in lane row 0, out of range elsewhere
  float pinf;                            // +inf, opaque to the compiler (max2)
};

// Buffer views of one pipeline run: chunks [start, start + count) of row b.
template <bool PER_LAYER>
__device__ __forceinline__ Ctx make_ctx(const uint8_t* comp_k, int B, int64_t N, int b, int64_t start, int64_t count,
                                        int lane, float* scores, float* per_layer) {
  Ctx cx;
  cx.c = lane & 15;
  cx.g = lane >> 4;
  cx.lane_rec_off = (uint32_t)(cx.c * kRecord + 32 * cx.g);
  cx.lane_scale_off = (uint32_t)(cx.c * kRecord + kHeadDim);
  cx.lane_out_off = cx.g == 0 ? (uint32_t)(cx.c * 4) : kDropOffset;
  cx.rec = comp_k + ((size_t)b * N + start) * kRecord;
  cx.out = scores + (size_t)b * N + start;
  cx.rec_bytes = (int32_t)(count * kRecord);
  cx.out_bytes = (int32_t)(count * 4);
  cx.count = (int32_t)count;
  cx.mask = nullptr;
  cx.lane_mask_off = lane < 4 ? (uint32_t)(4 * lane) : kDropOffset;
  cx.nib_shift = 4u * (uint32_t)(lane & 3);
  // Bytes beyond a row's valid chunks are zero in the mask, so a word may
  // cover them.
  cx.mask_words = (int32_t)idx::run_mask_words(start, count, N);
  cx.threshold = 0.f;
  cx.grp_chunk = 16 * kGroupTile[cx.g] + cx.c;
  cx.lane_grp_off = (uint32_t)(4 * cx.grp_chunk);
  cx.lane_grp_mask_off = cx.g == 0 ? (uint32_t)(4 * cx.c) : kDropOffset;
  {
    float inf = __builtin_huge_valf();
    asm volatile("" : "+s"(inf));
    cx.pinf = inf;
  }
#pragma unroll
  for (int l = 0; l < kLayers; ++l) {
    cx.lane_pl_off[l] = cx.g == kLayerRow[l] ? (uint32_t)(cx.c * 4) : kDropOffset;
    cx.pl[l] = PER_LAYER ? per_layer + ((size_t)l * B + b) * N + start : scores;
  }
  return cx;
}

// A buffer from byte `from` to `bytes` of a run's buffer (empty when `from`
// is past the end, or negative: the tile before the run's first).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int32_t bytes, int32_t from) {
  const int32_t left = from < 0 ? 0 : bytes - from;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)base + from), 0, left > 0 ? left : 0,
                                           kBufferWord3);
}

// Records of tile `tile` (>= 0) of the run.  The descriptor spans the whole
// run and the tile's byte offset goes in the scalar offset: on gfx950 a lane
// is in range when vector offset + scalar offset < size (checked on the GPU
// with in-bounds loads), so lanes past the run's end read zeros exactly as
// with a descriptor starting at the tile, and per tile only the offset
// changes (one scalar add, no new base address).
__device__ __forceinline__ void load_tile(const Ctx& cx, int tile, RawTile& t) {
  const int32_t from = tile * kTileBytes;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)cx.rec, 0, cx.rec_bytes, kBufferWord3);
  t.lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, cx.lane_rec_off, from, 0));
  t.hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, cx.lane_rec_off + 16, from, 0));
  t.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, cx.lane_scale_off, from, 0));
}

// Threshold mode folded into the score pass: the tile's 16 mask bytes,
// score > threshold, go out as four words from lanes 0..3, built from the
// compare mask (bit c is chunk c: lane l spreads bits 4l..4l+3 to the bytes
// of its word; chunks past the run give 0).  The score pipeline runs it one
// phase after the tile's scores (for tile i - 2 in the phase of tile i), so
// that it does not wait on the phase's own epilogue chain; the tile before
// the first (tile -1) writes nothing.
__device__ __forceinline__ void threshold_tile(const Ctx& cx, float e, int tile) {
  const int32_t n0 = tile * kTile;
  const int32_t tile_valid = n0 < 0 ? 0 : cx.count - n0;  // chunks of this tile inside the run (wave-uniform)
  const uint64_t keep = __ballot(e > cx.threshold && cx.c < tile_valid);
  const uint32_t nib = (uint32_t)(keep >> cx.nib_shift) & 0xfu;
  const uint32_t word = (nib * 0x204081u) & 0x01010101u;  // bit k -> byte k (a 24-bit multiply)
  __builtin_amdgcn_raw_buffer_store_b32(word, tile_rsrc(cx.mask, cx.mask_words, n0), cx.lane_mask_off, 0, 0);
}

// Ensemble and score store of one tile; returns the tile's ensemble scores
// (lane c and its copies in the other lane groups: chunk c).  u[l] is this
// lane's part of layer l's
// logit divided by |s| (as = |s|, the chunk's scale magnitude): the logit is
// |s| times the sum of u[l] over the four lane groups, and since |s| >= 0,
// max_l sigmoid(|s| T_l) = sigmoid(|s| max_l T_l) takes one sigmoid.  For
// the mean and per-layer outputs each lane row computes the sigmoid of the
// layer total it holds.
template <bool MEAN, bool PER_LAYER>
__device__ __forceinline__ float store_tile(const Ctx& cx, const float (&u)[kLayers], float as, int tile) {
  const int32_t to = tile * (kTile * 4);
  float e;
  if (MEAN || PER_LAYER) {
    // Row 3 holds 0 for the mean (its sigmoid, 1/2, is taken back out of
    // the sum) and layer 2 again for the max.
    const float sl = sigmoid(as * layer_totals(u, MEAN));
    e = MEAN ? (sum4rows(sl) - 0.5f) * (1.0f / 3.0f) : max4rows(sl, cx.pinf);
    if (PER_LAYER) {
#pragma unroll
      for (int l = 0; l < kLayers; ++l)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sl), tile_rsrc(cx.pl[l], PER_LAYER ? cx.out_bytes : 0, to),
                                              cx.lane_pl_off[l], 0, 0);
    }
  } else {
    e = sigmoid(as * max4rows(layer_totals(u, false), cx.pinf));
  }
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), tile_rsrc(cx.out, cx.out_bytes, to), cx.lane_out_off, 0, 0);
  return e;
}

// Four-tile groups of the scores-only outputs (the maximum and mean
// ensembles without per-layer scores).  Per tile, tile_rows gives each lane
// row's layer total times |s|, or for the mean its sigmoid (lane row 3 holds
// layer 2 again for the maximum, 0 for the mean); per group, group_scores
// reduces the rows of the four tiles together and takes one sigmoid for the
// maximum (|s| >= 0, so max_l |s| T_l = |s| max_l T_l, rounding included).
template <bool MEAN>
__device__ __forceinline__ float tile_rows(const float (&u)[kLayers], float as) {
  const float x = as * layer_totals(u, MEAN);
  return MEAN ? sigmoid(x) : x;
}
template <bool MEAN>
__device__ __forceinline__ float group_scores(const Ctx& cx, const float (&x)[4]) {
  const float r = reduce4<MEAN>(x[0], x[1], x[2], x[3], cx.pinf);
  return MEAN ? (r - 0.5f) * (1.0f / 3.0f) : sigmoid(r);
}
// Scores of the group of tiles tile0 .. tile0 + 3 (tile0 >= 0): one
// 256-byte store, addressed like load_tile's records (the run's descriptor,
// the group's offset in the scalar offset; stores past the run are dropped).
__device__ __forceinline__ void store_group(const Ctx& cx, float e, int tile0) {
  const int32_t from = tile0 * (kTile * 4);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)cx.out, 0, cx.out_bytes, kBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), r, cx.lane_grp_off, from, 0);
}
// Threshold mask of the group of tiles tile0 .. tile0 + 3 (64 bytes, 16
// words from lanes 0..15); a group before the run's first tile (tile0 < 0)
// writes nothing.  Ballot bit 16 g + c is group chunk 16 kGroupTile[g] + c:
// trading the middle two 16-bit fields puts the bits in chunk order, and
// lane c spreads bits 4c .. 4c + 3 to the bytes of its word.
__device__ __forceinline__ void threshold_group(const Ctx& cx, float e, int tile0) {
  const int32_t n0 = tile0 * kTile;
  // The run's mask descriptor with the group's offset in the scalar offset
  // (as in load_tile); empty for a group before the run.
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)cx.mask, 0, n0 < 0 ? 0 : cx.mask_words, kBufferWord3);
  uint64_t keep = __ballot(e > cx.threshold && n0 + cx.grp_chunk < cx.count);
  keep = (keep & 0xffff00000000ffffull) | ((keep >> 16) & 0xffff0000ull) | ((keep << 16) & 0xffff00000000ull);
  const uint32_t nib = (uint32_t)(keep >> (4 * cx.c)) & 0xfu;
  const uint32_t word = (nib * 0x204081u) & 0x01010101u;  // bit k -> byte k (a 24-bit multiply)
  __builtin_amdgcn_raw_buffer_store_b32(word, r, cx.lane_grp_mask_off, n0 < 0 ? 0 : n0, 0);
}

// The persistent grid's work split (idx::walk_runs): wave 4 blockIdx.x +
// (threadIdx.x / 64) of 4 gridDim.x waves scores its share of the tile list,
// one pipeline run per row it touches.
template <class Run>
__device__ __forceinline__ void walk_share(int B, int64_t N, const int32_t* __restrict__ valid_n,
                                           const int64_t* __restrict__ row_tiles,
                                           const int32_t* __restrict__ wave_row, int64_t total_tiles, Run&& run) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps descriptors scalar
  idx::walk_runs(4 * (int64_t)blockIdx.x + wave, 4 * (int64_t)gridDim.x, B, N, valid_n, row_tiles, wave_row,
                 total_tiles, run);
}

}  // namespace score
}  // namespace fm
