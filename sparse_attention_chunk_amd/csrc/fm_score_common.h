// Parts shared by the two score kernels (the f16-MFMA path in fm_score.hip
// and the fp8-MFMA path in fm_score_fp8.hip): record tiles and their loads,
// the per-lane buffer views of one pipeline run, the cross-lane head sum, the
// ensemble and store of a tile's scores, and the walk of a wave's share of
// the tile list.
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
constexpr int kTile = 16;                        // chunks per MFMA column tile
constexpr int kTileBytes = kTile * kRecord;      // 2112
constexpr int64_t kMaxSegTiles = 1 << 16;        // tiles per pipeline run: buffer offsets stay below 2^31
constexpr int kRing = 8;                         // register ring of record tiles
constexpr int kAhead = 6;                        // tile i + 6 is requested in the phase of tile i

// An offset past every buffer of one pipeline run (they hold at most
// 16 kMaxSegTiles + 8 tiles of records): the store is dropped by the range
// check, with no branch.
constexpr uint32_t kDropOffset = 0x40000000u;

// Sum over the four lane groups {l, l^16, l^32, l^48} (every lane gets it).
__device__ __forceinline__ float sum4groups(float v) {
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

struct RawTile {
  u32x4 lo, hi;  // this lane's 32 code bytes
  float s;       // the chunk's scale
};

struct Ctx {
  __amdgpu_buffer_rsrc_t rec;            // records of this wave's chunks; reads past them return 0
  __amdgpu_buffer_rsrc_t out;            // scores of this wave's chunks; writes past them are dropped
  __amdgpu_buffer_rsrc_t pl[kLayers];    // per-layer scores of this wave's chunks (when requested)
  uint32_t lane_rec_off;                 // 132 c + 32 g
  uint32_t lane_scale_off;               // 132 c + 128
  uint32_t lane_out_off;                 // 4 c in lane group 0, out of range elsewhere
  uint32_t lane_pl_off[kLayers];         // 4 c in lane group l, out of range elsewhere
  int c, g;
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
  cx.rec = __builtin_amdgcn_make_buffer_rsrc((void*)(comp_k + ((size_t)b * N + start) * kRecord), 0,
                                             (int)(count * kRecord), kBufferWord3);
  cx.out = __builtin_amdgcn_make_buffer_rsrc((void*)(scores + (size_t)b * N + start), 0, (int)(count * 4),
                                             kBufferWord3);
#pragma unroll
  for (int l = 0; l < kLayers; ++l) {
    cx.lane_pl_off[l] = cx.g == l ? (uint32_t)(cx.c * 4) : kDropOffset;
    cx.pl[l] = __builtin_amdgcn_make_buffer_rsrc(
        PER_LAYER ? (void*)(per_layer + ((size_t)l * B + b) * N + start) : (void*)scores, 0,
        PER_LAYER ? (int)(count * 4) : 0, kBufferWord3);
  }
  return cx;
}

// Offsets go in the per-lane voffset (the range check covers voffset).
__device__ __forceinline__ void load_tile(const Ctx& cx, int tile, RawTile& t) {
  const uint32_t so = (uint32_t)tile * kTileBytes;
  t.lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cx.rec, cx.lane_rec_off + so, 0, 0));
  t.hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cx.rec, cx.lane_rec_off + so + 16, 0, 0));
  t.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cx.rec, cx.lane_scale_off + so, 0, 0));
}

// Sigmoid, ensemble and store of one tile from the layers' logits t[l]
// (every lane holds its chunk's logits).
template <bool MEAN, bool PER_LAYER>
__device__ __forceinline__ void store_tile(const Ctx& cx, const float (&t)[kLayers], int tile) {
  float e;
  float sl[kLayers];
  if (MEAN || PER_LAYER) {
#pragma unroll
    for (int l = 0; l < kLayers; ++l) sl[l] = sigmoid(t[l]);
    e = MEAN ? (sl[0] + sl[1] + sl[2]) * (1.0f / 3.0f) : fmaxf(fmaxf(sl[0], sl[1]), sl[2]);
  } else {
    // max_l sigmoid(t_l) = sigmoid(max_l t_l): one sigmoid.
    e = sigmoid(fmaxf(fmaxf(t[0], t[1]), t[2]));
  }
  const uint32_t to = (uint32_t)tile * (kTile * 4);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), cx.out, cx.lane_out_off + to, 0, 0);
  if (PER_LAYER) {
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sl[l]), cx.pl[l], cx.lane_pl_off[l] + to, 0, 0);
  }
}

// The persistent grid's work split: the valid tiles of all rows, in
// row-major order, are cut into equal contiguous shares, one per wave (4
// waves per block): with row_tiles (prefix of the rows' valid tile counts,
// from the plan kernel) when rows are ragged, else every row has
// ceil(N / 16) tiles.  A share may end in the next row (or, for short rows,
// several rows later): each row's part is its own pipeline run,
// run(b, start, count), at most kMaxSegTiles tiles long.
template <class Run>
__device__ __forceinline__ void walk_share(int B, int64_t N, const int32_t* __restrict__ valid_n,
                                           const int64_t* __restrict__ row_tiles,
                                           const int32_t* __restrict__ wave_row, int64_t total_tiles, Run&& run) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps descriptors scalar
  const int64_t waves = 4 * (int64_t)gridDim.x;
  const int64_t gw = 4 * (int64_t)blockIdx.x + wave;
  const int64_t total = row_tiles ? row_tiles[B] : total_tiles;
  int64_t t = gw * total / waves;
  const int64_t t_end = (gw + 1) * total / waves;
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
      int64_t vn = N;
      if (valid_n) {
        const int64_t v = valid_n[b];
        vn = v < 0 ? 0 : (v > N ? N : v);
      }
      const int64_t start = (t - first) * kTile;
      const int64_t end = run_end - first == last - first ? vn : (run_end - first) * kTile;
      run(b, start, end - start);
    }
    t = run_end;
    if (t >= last) {
      ++b;
      first = last;
    }
  }
}

}  // namespace score
}  // namespace fm
