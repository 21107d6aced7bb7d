// Keep masks (FlashMemory DS-V4 Retriever README, "Usage": select_topk with
// top_k=... or threshold=...; "Inference flow": keep_mask = top-K of the
// scores, or sigmoid > thresh).
//
// Top-K is an exact per-row selection on order-preserving 32-bit keys of the
// fp32 scores; ties at the K-th key go to the lowest chunk indices, which
// makes the mask unique.  Two kernels per call:
//   1. scan (every chunk, all compute units): the mask bytes (0, or 1 for
//      every valid chunk of a row whose K keeps them all) and a word per
//      tile of the row: the histogram bins of the tile's three largest
//      scores and the positions of the largest two.  A tile is 16, 32 or 64
//      chunks, the largest that still leaves 4 K tiles in the row;
//   2. finish (one block per row): the histogram of the row's tile maxima
//      gives the bin c of the K-th largest tile maximum L (bin 0 when the
//      row has fewer than K tiles).  The K tiles with the largest maxima hold
//      K distinct chunks scoring at least L, so the K-th largest score is
//      >= L: every chunk of the top K is in bin c or above, and so is its
//      tile's maximum.  Of a tile whose maximum is in bin c or above, only
//      the chunks of its largest scores down to the first one below bin c
//      can be: one or two known chunks, or, when the third largest is in bin
//      c or above too, all the tile's chunks.  Those in bin c or above
//      (about K) are the candidates.  One more histogram, of the candidates'
//      keys between their smallest and largest, gives the bin of the K-th
//      largest candidate: the candidates above it are kept, those in it are
//      ranked (key descending, index ascending) for the rest.
// When the listed chunks or the candidates overflow LDS (many equal or
// nearly equal scores), the finish selects exactly over the whole row with
// radix passes instead, so the result is always the exact top-K.  Short
// rows (below) skip the scan: one launch selects each row with radix passes
// over its keys held in registers.
#include "fm_radix.h"

namespace fm {
namespace {

using namespace radix;

__device__ inline int64_t row_valid(const int32_t* valid_n, int b, int64_t N) {
  if (!valid_n) return N;
  const int64_t v = valid_n[b];
  return v < 0 ? 0 : (v > N ? N : v);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 16;             // chunks per scan thread (a tile is 1, 2 or 4 of these)
constexpr int kScanThreads = 256;
constexpr int kScanSlice = kScanThreads * kSub;
constexpr int kFinishThreads = 512;  // 17.6 us per call at B=30, N=262144, K=512 (256: 19.3, 1024: 17.8)
constexpr int kFinishRegPairs = 4;   // pairs of tile words per thread read into registers (4096 tiles a row)
constexpr int kFinishRegEntries = 2; // listed chunks per thread held in registers (1024 a row)
constexpr int kFinishList = 4096;    // listed chunks held in LDS
constexpr int kFinishFull = 256;     // tiles listed whole
constexpr int kFinishCand = 4096;    // candidates held in LDS
constexpr float kHistScale = kSelBins - 0.25f;
constexpr int kRawBuffer = 0x00020000;         // raw buffer, 32-bit data format
constexpr uint32_t kOutOfRange = 0x40000000u;  // a byte offset past every buffer here: loads give 0
constexpr uint32_t kNone = 0xffffffffu;        // no chunk

// Histogram bin of a score, floor(score (kSelBins - 1/4)) clamped to
// [0, kSelBins): non-decreasing in the score, one bin per 1/2048 of [0, 1]
// where sigmoid scores lie.
__device__ __forceinline__ int score_bin(float e) {
  const float x = e * kHistScale;
  return !(x > 0.f) ? 0 : (x >= (float)(kSelBins - 1) ? kSelBins - 1 : (int)x);  // NaN: bin 0
}
// The float whose order_key is k.
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// The bin of an entry's key; key 0 (no order_key of a score is 0) marks an
// entry that is never chosen and sits in bin 0.
__device__ __forceinline__ int key_bin(uint32_t k) { return k == 0 ? 0 : score_bin(key_float(k)); }
// key_bin(k) >= c, for c in [0, kSelBins): x >= c when c >= 1, as the
// integer part of x > 0 is at least c exactly when x is.
__device__ __forceinline__ bool key_at_least(uint32_t k, int c) {
  return c == 0 || (k != 0 && key_float(k) * kHistScale >= (float)c);
}

// log2 of the tile's kSub-chunk parts in a row of vn chunks (0..2): the
// largest leaving at least 4 K tiles.
using idx::tile_shift;
static_assert(kSub == idx::kSelSub, "scan part size");

// Tile word: x bits 0-10 the largest key's bin, 11-16 its position in the
// tile, 17-27 the second largest's bin; y bits 0-5 the second largest's
// position, 6-16 the third largest's bin (bin 0 where there is none), 17-23
// the tile's entries with a key (not 0).  Ties count as separate entries.
__device__ __forceinline__ int tw_bin1(uint2 w) { return (int)(w.x & 0x7ffu); }
__device__ __forceinline__ uint32_t tw_pos1(uint2 w) { return (w.x >> 11) & 0x3fu; }
__device__ __forceinline__ int tw_bin2(uint2 w) { return (int)((w.x >> 17) & 0x7ffu); }
__device__ __forceinline__ uint32_t tw_pos2(uint2 w) { return w.y & 0x3fu; }
__device__ __forceinline__ int tw_bin3(uint2 w) { return (int)((w.y >> 6) & 0x7ffu); }
__device__ __forceinline__ uint32_t tw_count(uint2 w) { return (w.y >> 17) & 0x7fu; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)bytes, kRawBuffer);
}

// The three largest keys of a set of entries: m1 >= m2 >= m3 (0 where
// there is none), positions of the first two, and the entries with a key.
struct Top3 {
  uint32_t m1, m2, m3;
  uint32_t p1, p2, n;
};

__device__ __forceinline__ void top3_take(Top3& a, uint32_t v, uint32_t pos) {
  const bool gt1 = v > a.m1;
  const bool gt2 = v > a.m2;
  a.n += v != 0 ? 1u : 0u;
  a.m3 = gt2 ? a.m2 : max(a.m3, v);
  a.m2 = gt1 ? a.m1 : (gt2 ? v : a.m2);
  a.p2 = gt1 ? a.p1 : (gt2 ? pos : a.p2);
  a.m1 = gt1 ? v : a.m1;
  a.p1 = gt1 ? pos : a.p1;
}

// The three largest of the union of two disjoint sets' (ties to the lower
// position).
__device__ __forceinline__ Top3 top3_merge(const Top3& a, const Top3& b) {
  const bool af = a.m1 > b.m1 || (a.m1 == b.m1 && a.p1 < b.p1);  // a holds the largest
  const uint32_t w1 = af ? a.m1 : b.m1, w2 = af ? a.m2 : b.m2, w3 = af ? a.m3 : b.m3;
  const uint32_t wp1 = af ? a.p1 : b.p1, wp2 = af ? a.p2 : b.p2;
  const uint32_t l1 = af ? b.m1 : a.m1, l2 = af ? b.m2 : a.m2;
  const uint32_t lp1 = af ? b.p1 : a.p1;
  const bool w_second = w2 > l1 || (w2 == l1 && wp2 < lp1);
  Top3 r;
  r.m1 = w1;
  r.p1 = wp1;
  r.m2 = w_second ? w2 : l1;
  r.p2 = w_second ? wp2 : lp1;
  r.m3 = w_second ? max(w3, l1) : max(w2, l2);
  r.n = a.n + b.n;
  return r;
}

// Merges the Top3 of the 2^s adjacent lanes of a tile (lane groups of 2^s),
// then encodes the tile word (every lane of the group holds it).
__device__ __forceinline__ uint2 tile_word(Top3 a, int s) {
  for (int i = 0; i < s; ++i) {
    Top3 o;
    o.m1 = (uint32_t)__shfl_xor((int)a.m1, 1 << i);
    o.m2 = (uint32_t)__shfl_xor((int)a.m2, 1 << i);
    o.m3 = (uint32_t)__shfl_xor((int)a.m3, 1 << i);
    o.p1 = (uint32_t)__shfl_xor((int)a.p1, 1 << i);
    o.p2 = (uint32_t)__shfl_xor((int)a.p2, 1 << i);
    o.n = (uint32_t)__shfl_xor((int)a.n, 1 << i);
    a = top3_merge(a, o);
  }
  return make_uint2((uint32_t)key_bin(a.m1) | (a.p1 << 11) | ((uint32_t)key_bin(a.m2) << 17),
                    a.p2 | ((uint32_t)key_bin(a.m3) << 6) | (a.n << 17));
}

// 1. Mask bytes and tile words.  grid = (ceil(N / kScanSlice), B), block =
// kScanThreads; thread t covers the 16 chunks of part g = blockIdx.x 256 + t,
// and the 2^s threads of a tile (adjacent lanes) merge their parts.
__global__ __launch_bounds__(kScanThreads) void topk_scan_kernel(const float* __restrict__ scores, int64_t N,
                                                                 const int32_t* __restrict__ valid_n, int32_t top_k,
                                                                 uint2* __restrict__ tile_info,
                                                                 uint8_t* __restrict__ mask) {
  const int b = blockIdx.y;
  const int64_t vn = row_valid(valid_n, b, N);
  const int64_t g = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
  const int64_t n0 = g * kSub;
  const float* row = scores + (size_t)b * N;
  uint8_t* mrow = mask + (size_t)b * N;
  const bool keep_all = (int64_t)top_k >= vn;  // also vn = 0
  // Rows the finish selects in (uniform over the block): the tile words.
  if (!keep_all && top_k > 0 && (int64_t)blockIdx.x * kScanSlice < vn) {
    const int s = tile_shift(vn, top_k);
    const uint32_t p0 = (uint32_t)(g & ((1 << s) - 1)) * kSub;  // the part's first position in its tile
    Top3 a = {0u, 0u, 0u, p0, p0, 0u};  // parts past vn hold no entry
    if (n0 + kSub <= vn && ((((uintptr_t)(row + n0)) & 15) == 0)) {
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *(const float4*)(row + n0 + 4 * q);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        top3_take(a, order_key(v[q].x), p0 + 4 * q);
        top3_take(a, order_key(v[q].y), p0 + 4 * q + 1);
        top3_take(a, order_key(v[q].z), p0 + 4 * q + 2);
        top3_take(a, order_key(v[q].w), p0 + 4 * q + 3);
      }
    } else {
      for (int j = 0; j < kSub && n0 + j < vn; ++j) top3_take(a, order_key(row[n0 + j]), p0 + j);
    }
    const uint2 word = tile_word(a, s);
    const int64_t tile = idx::scan_tile_written(g, s, vn);
    if (tile >= 0) tile_info[(size_t)b * tile_info_stride(N) + tile] = word;
  }
  if (n0 >= N) return;
  const uint8_t keep = keep_all ? 1 : 0;
  if (n0 + kSub <= N && ((((uintptr_t)(mrow + n0)) & 15) == 0) && (!keep_all || n0 + kSub <= vn)) {
    const uint32_t wv = keep * 0x01010101u;
    *(uint4*)(mrow + n0) = make_uint4(wv, wv, wv, wv);
  } else {
    for (int j = 0; j < kSub && n0 + j < N; ++j) mrow[n0 + j] = n0 + j < vn ? keep : 0;
  }
}

// Exclusive block-wide prefix sum of v; *total receives the sum.  Ends with
// a barrier, so s_wtot may be reused right after.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wtot, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_prefix_sum(v);
  if (lane == 63) s_wtot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kFinishThreads / 64; ++w) {
    const uint32_t x = s_wtot[w];
    before += w < wave ? x : 0u;
    all += x;
  }
  *total = all;
  __syncthreads();
  return before + incl - v;
}

// 1b. Keys and tile words of subset lists (the per-step top-K over the
// resident set).  grid = (ceil(cap / kSubScanSlice), B), block =
// kScanThreads; thread t covers list positions 4 g .. 4 g + 3, g =
// blockIdx.x 256 + t (many threads, so many index -> score gathers in
// flight), and the 4 2^s threads of a tile merge their parts.  The key of a
// position is the order_key of its chunk's score, or 0 when the position is
// past the row's list or its chunk is outside [0, N).
constexpr int kSubPart = 4;
constexpr int kSubScanSlice = kScanThreads * kSubPart;
__global__ __launch_bounds__(kScanThreads) void subset_scan_kernel(const float* __restrict__ scores, int64_t N,
                                                                   const int32_t* __restrict__ subset,
                                                                   const int32_t* __restrict__ n_subset,
                                                                   int32_t cap, int32_t top_k,
                                                                   uint32_t* __restrict__ keys,
                                                                   uint2* __restrict__ tile_info) {
  const int b = blockIdx.y;
  const int64_t n64 = n_subset ? (int64_t)n_subset[b] : (int64_t)cap;
  const uint32_t n = (uint32_t)(n64 < 0 ? 0 : (n64 > cap ? cap : n64));
  if (top_k == 0 || (uint32_t)blockIdx.x * kSubScanSlice >= n) return;  // uniform over the block
  const uint32_t g = blockIdx.x * kScanThreads + threadIdx.x;
  const uint32_t p0 = g * kSubPart;
  const __amdgpu_buffer_rsrc_t rs = buffer(subset + (size_t)b * cap, 4 * (int64_t)n);
  const __amdgpu_buffer_rsrc_t rv = buffer(scores + (size_t)b * N, N < 0x20000000 ? 4 * N : 0x7fffffff);
  const u32x4 iv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4u * p0, 0, 0));
  const int32_t idx[kSubPart] = {(int32_t)iv.x, (int32_t)iv.y, (int32_t)iv.z, (int32_t)iv.w};
  uint32_t k[kSubPart];
#pragma unroll
  for (int j = 0; j < kSubPart; ++j) {
    const bool ok = p0 + j < n && idx[j] >= 0 && (int64_t)idx[j] < N;
    const float v = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rv, ok ? 4u * (uint32_t)idx[j] : kOutOfRange, 0, 0));
    k[j] = ok ? order_key(v) : 0u;
  }
  const int s = tile_shift(n, top_k);
  const int m = s + 2;                                  // log2 of the parts per tile
  const uint32_t pt = (g & ((1u << m) - 1)) * kSubPart;  // the part's first position in its tile
  Top3 a = {0u, 0u, 0u, pt, pt, 0u};
#pragma unroll
  for (int j = 0; j < kSubPart; ++j) top3_take(a, k[j], pt + j);
  const uint2 word = tile_word(a, m);
  uint32_t* krow = keys + (size_t)b * kSubFastCap;
  if (p0 < n) *(uint4*)(krow + p0) = make_uint4(k[0], k[1], k[2], k[3]);
  const uint32_t tile = g >> m;
  if (pt == 0 && (tile << (4 + s)) < n) tile_info[(size_t)b * (kSubFastCap / kSub) + tile] = word;
}

// 2. Exact top-K of each row.  grid = B, block = kFinishThreads.  SUBSET:
// the entries are the positions of the row's subset list (keys staged by
// subset_scan_kernel; the chosen ones written as chunk indices in list
// order to out, their number to n_out); else the row's chunks (keys from
// the scores; the chosen ones' mask bytes set).
template <bool SUBSET>
__global__ __launch_bounds__(kFinishThreads) void topk_finish_kernel(
    const float* __restrict__ scores, int64_t N, const int32_t* __restrict__ valid_n, int32_t top_k,
    const uint2* __restrict__ tile_info, uint8_t* __restrict__ mask, const uint32_t* __restrict__ keys,
    const int32_t* __restrict__ subset, const int32_t* __restrict__ n_subset, int32_t cap, int32_t* __restrict__ out,
    int32_t* __restrict__ n_out) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ __attribute__((aligned(16))) uint32_t h[2 * kSelBins];
  __shared__ uint32_t s_e[kFinishList];
  __shared__ uint32_t s_f[kFinishFull];
  __shared__ uint2 s_c[kFinishCand];
  __shared__ uint2 s_r[kFinishThreads];
  __shared__ uint32_t s_wtot[kFinishThreads / 64];
  __shared__ uint32_t s_mm[2 * (kFinishThreads / 64)];
  __shared__ uint32_t s_out[3];
  __shared__ uint32_t s_bits[SUBSET ? kSubFastCap / 32 : 1];  // chosen list positions

  // vn: the row's entries (chunks below valid_n, or list positions).
  int64_t vn;
  if (SUBSET) {
    const int64_t n64 = n_subset ? (int64_t)n_subset[b] : (int64_t)cap;
    vn = n64 < 0 ? 0 : (n64 > cap ? cap : n64);
    if (top_k == 0 || vn == 0) {
      if (t == 0) n_out[b] = 0;
      return;
    }
  } else {
    vn = row_valid(valid_n, b, N);
    if (top_k == 0 || (int64_t)top_k >= vn) return;  // the scan wrote the whole mask
  }
  uint8_t* mrow = mask + (SUBSET ? 0 : (size_t)b * N);
  const float* row = scores + (size_t)b * N;
  const uint32_t* krow = keys + (SUBSET ? (size_t)b * kSubFastCap : 0);
  uint32_t K = (uint32_t)top_k;
  const uint32_t vn32 = (uint32_t)vn;  // below 2^26
  const __amdgpu_buffer_rsrc_t rr = SUBSET ? buffer(krow, vn * 4) : buffer(row, vn * 4);
  // The key of entry n (loads past vn give key 0 / score 0, never used).
  auto key_of = [&](uint32_t n) -> uint32_t {
    const uint32_t raw = __builtin_amdgcn_raw_buffer_load_b32(rr, n != kNone ? 4u * n : kOutOfRange, 0, 0);
    return SUBSET ? raw : order_key(__uint_as_float(raw));
  };
  auto emit = [&](uint32_t n) {
    if (SUBSET) atomicOr(&s_bits[n >> 5], 1u << (n & 31));
    else mrow[n] = 1;
  };

  // Tile words: thread t holds tiles 512 (j / 2) + 2 t + j % 2 (16-byte
  // loads through a descriptor over the row's slot, a multiple of 16 bytes:
  // zeros past it); their maxima are counted in the row's histogram.
  const int s = tile_shift(vn, top_k);
  const int lt = 4 + s;  // log2 of the tile's entries
  const uint32_t nt = (uint32_t)idx::finish_tiles(vn, s);
  const int64_t tstride = SUBSET ? kSubFastCap / kSub : tile_info_stride(N);
  const uint2* irow = tile_info + (size_t)b * tstride;
  const __amdgpu_buffer_rsrc_t ir = buffer(irow, tstride * 8);
  constexpr int kRegTiles = 2 * kFinishRegPairs;
  uint2 info[kRegTiles];
#pragma unroll
  for (int j = 0; j < kFinishRegPairs; ++j) {
    const u32x4 v = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(ir, 16u * (kFinishThreads * j + t), 0, 0));
    info[2 * j] = make_uint2(v.x, v.y);
    info[2 * j + 1] = make_uint2(v.z, v.w);
  }
  auto tile_of = [&](int j) { return (uint32_t)(2 * kFinishThreads * (j >> 1) + 2 * t + (j & 1)); };
  constexpr uint32_t kBlockTiles = (uint32_t)kRegTiles * kFinishThreads;
  clear_bins<kFinishThreads>(h);
  if (SUBSET)
    for (int i = t; i < kSubFastCap / 32; i += kFinishThreads) s_bits[i] = 0u;
  __syncthreads();
  uint32_t counted = 0;  // entries with a key in this thread's tiles
#pragma unroll
  for (int j = 0; j < kRegTiles; ++j)
    if (tile_of(j) < nt) {
      atomicAdd(&h[tw_bin1(info[j])], 1u);
      counted += tw_count(info[j]);
    }
  for (uint32_t i = kBlockTiles + t; i < nt; i += kFinishThreads) {
    const uint2 w = irow[i];
    atomicAdd(&h[tw_bin1(w)], 1u);
    counted += tw_count(w);
  }
  __syncthreads();
  if (SUBSET) {
    // The chosen number: K, or every entry with a key when there are fewer.
    uint32_t n_keyed;
    (void)block_excl_scan(counted, s_wtot, &n_keyed);
    if (K >= n_keyed) {
      for (uint32_t n = t; n < vn32; n += kFinishThreads)
        if (key_of(n) != 0) emit(n);
      K = n_keyed;
      goto write_out;
    }
  }
  {
  int c = 0;
  if (K <= nt) {
    block_find<kFinishThreads>(h, K, s_wtot, s_out, true);
    c = (int)s_out[0];
  }
  // The listed chunks of each tile whose maximum is in bin c or above: its
  // largest one or two (s_e), or, when its third largest is in bin c or
  // above too, the whole tile (s_f).  Each thread classifies its register
  // tiles without branches (2 bits each: 0 none, 1 the largest chunk, 2 the
  // largest two, 3 the whole tile) and counts its entries; one scan places
  // both lists (counts in the low and high 16 bits), and a second pass over
  // the same registers writes the thread's entries in tile order.
  uint32_t ne = 0, nf = 0;
  {
    uint32_t cnt = 0, kinds = 0;
#pragma unroll
    for (int j = 0; j < kRegTiles; ++j) {
      const uint2 w = info[j];
      const bool q = tile_of(j) < nt && tw_bin1(w) >= c;
      const uint32_t k = !q ? 0u : (tw_bin2(w) < c ? 1u : (tw_bin3(w) < c ? 2u : 3u));
      kinds |= k << (2 * j);
      cnt += k == 3u ? 0x10000u : k;
    }
    uint32_t tot;
    const uint32_t pos = block_excl_scan(cnt, s_wtot, &tot);
    ne = tot & 0xffffu;
    nf = tot >> 16;
    uint32_t pe = pos & 0xffffu, pf = pos >> 16;
#pragma unroll
    for (int j = 0; j < kRegTiles; ++j) {
      const uint32_t k = (kinds >> (2 * j)) & 3u;
      if (k != 0u) {
        const uint2 w = info[j];
        const uint32_t tile = tile_of(j);
        const uint32_t first = tile << lt;
        if (k == 3u) {
          if (pf < (uint32_t)kFinishFull) s_f[pf] = tile;
          ++pf;
        } else {
          if (pe < (uint32_t)kFinishList) s_e[pe] = first + tw_pos1(w);
          if (k == 2u && pe + 1 < (uint32_t)kFinishList) s_e[pe + 1] = first + tw_pos2(w);
          pe += k;
        }
      }
    }
  }
  for (uint32_t base = kBlockTiles; base < nt; base += kFinishThreads) {  // rows of more than kBlockTiles tiles
    const uint32_t i = base + t;
    const uint2 w = i < nt ? irow[i] : make_uint2(0u, 0u);
    const bool q = i < nt && tw_bin1(w) >= c;
    const uint32_t cnt = q ? (tw_bin2(w) < c ? 1u : (tw_bin3(w) < c ? 2u : 0x10000u)) : 0u;
    uint32_t tot;
    const uint32_t pos = block_excl_scan(cnt, s_wtot, &tot);
    const uint32_t pe = ne + (pos & 0xffffu), pf = nf + (pos >> 16);
    if (q) {
      const uint32_t first = i << lt;
      if (cnt < 0x10000u) {
        if (pe < (uint32_t)kFinishList) s_e[pe] = first + tw_pos1(w);
        if (cnt == 2u && pe + 1 < (uint32_t)kFinishList) s_e[pe + 1] = first + tw_pos2(w);
      } else if (pf < (uint32_t)kFinishFull) {
        s_f[pf] = i;
      }
    }
    ne += tot & 0xffffu;
    nf += tot >> 16;
  }
  __syncthreads();  // s_e, s_f complete

  if (ne <= (uint32_t)kFinishList && nf <= (uint32_t)kFinishFull) {
    // Listed entry x: s_e[x], then the chunks of the whole tiles in order.
    const uint32_t total = ne + (nf << lt);
    auto entry = [&](uint32_t x) -> uint32_t {
      if (x < ne) return s_e[x];
      const uint32_t y = x - ne;
      return (s_f[y >> lt] << lt) + (y & ((1u << lt) - 1));
    };
    // The candidates: listed entries with a key in bin c or above.
    auto final_select = [&](auto each) {
      // Bins of the keys between the smallest and the largest candidate:
      // (key - kmin) >> sh < kSelBins.
      const int lane = t & 63;
      const int wave = t >> 6;
      uint32_t kmin = 0xffffffffu, kmax = 0u;
      each([&](uint2 e) {
        kmin = e.x < kmin ? e.x : kmin;
        kmax = e.x > kmax ? e.x : kmax;
      });
      kmin = wave_min_u32(kmin);
      kmax = wave_max_u32(kmax);
      if (lane == 0) {
        s_mm[2 * wave] = kmin;
        s_mm[2 * wave + 1] = kmax;
      }
      clear_bins<kFinishThreads>(h);
      __syncthreads();
      kmin = 0xffffffffu;
      kmax = 0u;
#pragma unroll
      for (int w = 0; w < kFinishThreads / 64; ++w) {
        kmin = s_mm[2 * w] < kmin ? s_mm[2 * w] : kmin;
        kmax = s_mm[2 * w + 1] > kmax ? s_mm[2 * w + 1] : kmax;
      }
      const uint32_t span = kmax - kmin;
      const int width = span ? 32 - __builtin_clz(span) : 0;  // bits of the largest offset
      const int sh = width > 11 ? width - 11 : 0;
      each([&](uint2 e) { atomicAdd(&h[(e.x - kmin) >> sh], 1u); });
      __syncthreads();
      block_find<kFinishThreads>(h, K, s_wtot, s_out, true);
      const uint32_t c2 = s_out[0];
      const uint32_t need = K - s_out[1];  // of the candidates in bin c2
      // Those above bin c2 are kept; those in it are listed in s_r.
      uint32_t mine = 0;
      each([&](uint2 e) { mine += ((e.x - kmin) >> sh) == c2 ? 1u : 0u; });
      uint32_t in_c2;
      uint32_t pos = block_excl_scan(mine, s_wtot, &in_c2);
      each([&](uint2 e) {
        const uint32_t bn = (e.x - kmin) >> sh;
        if (bn > c2) emit(e.y);
        if (bn == c2) {
          if (pos < (uint32_t)kFinishThreads) s_r[pos] = e;
          ++pos;
        }
      });
      __syncthreads();  // s_r complete
      if (in_c2 <= (uint32_t)kFinishThreads) {
        if ((uint32_t)t < in_c2) {
          const uint2 me = s_r[t];
          uint32_t rank = 0;
          for (uint32_t j = 0; j < in_c2; ++j) {
            const uint2 o = s_r[j];
            rank += (o.x > me.x || (o.x == me.x && o.y < me.y)) ? 1u : 0u;
          }
          if (rank < need) emit(me.y);
        }
      } else {
        auto in_bin = [&](auto f) {
          each([&](uint2 e) {
            if (((e.x - kmin) >> sh) == c2) f(e);
          });
        };
        uint32_t T, last;
        radix_select<kFinishThreads>(in_bin, need, index_bits(vn), h, s_wtot, s_out, &T, &last);
        in_bin([&](uint2 e) {
          if (e.x > T || (e.x == T && e.y <= last)) emit(e.y);
        });
      }
    };
    if (total <= (uint32_t)(kFinishThreads * kFinishRegEntries)) {
      // Each thread holds its listed chunks in registers.
      uint32_t n[kFinishRegEntries];
      uint32_t e[kFinishRegEntries];
#pragma unroll
      for (int r = 0; r < kFinishRegEntries; ++r) {
        const uint32_t x = t + r * kFinishThreads;
        n[r] = x < total ? entry(x) : kNone;
      }
#pragma unroll
      for (int r = 0; r < kFinishRegEntries; ++r) e[r] = key_of(n[r]);
      uint2 cand[kFinishRegEntries];
      bool ok[kFinishRegEntries];
#pragma unroll
      for (int r = 0; r < kFinishRegEntries; ++r) {
        ok[r] = n[r] < vn32 && e[r] != 0 && key_at_least(e[r], c);
        cand[r] = make_uint2(e[r], n[r]);
      }
      final_select([&](auto f) {
#pragma unroll
        for (int r = 0; r < kFinishRegEntries; ++r)
          if (ok[r]) f(cand[r]);
      });
      goto write_out;
    }
    // More listed chunks: the candidates go to LDS first.
    uint32_t nc = 0;
    for (uint32_t base = 0; base < total; base += kFinishThreads * 4) {
      uint32_t n[4];
      uint32_t e[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t x = base + t + r * kFinishThreads;
        n[r] = x < total ? entry(x) : kNone;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) e[r] = key_of(n[r]);
      uint32_t okb = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n[r] < vn32 && e[r] != 0 && key_at_least(e[r], c)) okb |= 1u << r;
      uint32_t tot;
      uint32_t pos = nc + block_excl_scan(__popc(okb), s_wtot, &tot);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (okb & (1u << r)) {
          if (pos < (uint32_t)kFinishCand) s_c[pos] = make_uint2(e[r], n[r]);
          ++pos;
        }
      nc += tot;
    }
    __syncthreads();  // s_c complete
    if (nc <= (uint32_t)kFinishCand) {
      final_select([&](auto f) {
        for (uint32_t i = t; i < nc; i += kFinishThreads) f(s_c[i]);
      });
      goto write_out;
    }
  }
  // Too many equal or nearly equal keys for LDS: exact selection over all
  // the row's entries (nothing has been chosen yet).
  {
    auto each = [&](auto f) {
      for (uint32_t n = t; n < vn32; n += kFinishThreads) {
        const uint32_t k = key_of(n);
        if (!SUBSET || k != 0) f(make_uint2(k, n));
      }
    };
    uint32_t T, last;
    radix_select<kFinishThreads>(each, K, index_bits(vn), h, s_wtot, s_out, &T, &last);
    each([&](uint2 e) {
      if (e.x > T || (e.x == T && e.y <= last)) emit(e.y);
    });
  }
  }
write_out:
  if (SUBSET) {
    // The chosen positions in list order: thread t holds bitmap words 4 t ..
    // 4 t + 3; a scan of their counts gives each one's place in out.
    __syncthreads();
    uint32_t w4[4], cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int wi = 4 * t + q;
      w4[q] = wi < kSubFastCap / 32 ? s_bits[wi] : 0u;
      cnt += __popc(w4[q]);
    }
    uint32_t tot;
    uint32_t pos = block_excl_scan(cnt, s_wtot, &tot);
    const int32_t* srow = subset + (size_t)b * cap;
    int32_t* orow = out + (size_t)b * top_k;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t bits = w4[q];
      while (bits) {
        const uint32_t p = 32u * (4 * t + q) + __builtin_ctz(bits);
        bits &= bits - 1;
        if (pos < (uint32_t)top_k) orow[pos] = srow[p];
        ++pos;
      }
    }
    if (t == 0) n_out[b] = (int32_t)K;
  }
}

// Top-K of short rows in one launch instead of scan +
// finish: one block per row loads the row's keys into registers once (all
// loads in flight together), selects exactly over them with radix passes and
// then writes each mask byte of the row once.  The same chunks as the
// two-kernel path: keys above the K-th key T, and of those equal to T the
// ones up to `last` (ties to the lowest indices).
// Rows (lists) of up to kShortRow entries always take it (16 keys per
// thread); up to kShortRowMax (32 keys per thread) when they hold fewer than
// 18 K entries.  There the scan + finish path has too few tiles per K: the
// K-th tile maximum cuts almost nothing, the listed chunks overflow LDS and
// the finish falls back to radix passes that re-read the row (25 us at
// B=30, N=8193, K=512, against 8-10 us on either side).
constexpr int64_t kShortRow = 8192;
constexpr int64_t kShortRowMax = 16384;
static_assert(kShortRow % kFinishThreads == 0 && kShortRowMax % kFinishThreads == 0, "rows split evenly");
__host__ __device__ constexpr int short_per(int64_t n, int32_t top_k) {
  return n <= kShortRow ? (int)(kShortRow / kFinishThreads)
                        : (n <= kShortRowMax && n < 18 * (int64_t)top_k ? (int)(kShortRowMax / kFinishThreads) : 0);
}
template <int kShortPer>
__global__ __launch_bounds__(kFinishThreads) void topk_short_kernel(const float* __restrict__ scores, int64_t N,
                                                                    const int32_t* __restrict__ valid_n,
                                                                    int32_t top_k, uint8_t* __restrict__ mask) {
  __shared__ __attribute__((aligned(16))) uint32_t h[2 * kSelBins];
  __shared__ uint32_t s_wtot[kFinishThreads / 64];
  __shared__ uint32_t s_out[3];
  const int b = blockIdx.x;
  const uint32_t t = threadIdx.x;
  const int64_t vn = row_valid(valid_n, b, N);
  const float* row = scores + (size_t)b * N;
  uint8_t* mrow = mask + (size_t)b * N;
  const uint32_t n_all = (uint32_t)N, vn32 = (uint32_t)vn;  // N <= kShortPer kFinishThreads
  if (top_k == 0 || (int64_t)top_k >= vn) {  // uniform over the block: nothing or every valid chunk
    const uint8_t keep = top_k > 0 ? 1 : 0;
    for (uint32_t n = t; n < n_all; n += kFinishThreads) mrow[n] = n < vn32 ? keep : 0;
    return;
  }
  // Entry j of thread t is chunk t + j kFinishThreads.
  uint32_t keys[kShortPer];
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) {
    const uint32_t n = t + (uint32_t)j * kFinishThreads;
    keys[j] = n < vn32 ? order_key(row[n]) : 0u;
  }
  auto each = [&](auto f) {
#pragma unroll
    for (int j = 0; j < kShortPer; ++j) {
      const uint32_t n = t + (uint32_t)j * kFinishThreads;
      if (n < vn32) f(make_uint2(keys[j], n));
    }
  };
  uint32_t T, last;
  radix_select<kFinishThreads>(each, (uint32_t)top_k, index_bits(vn), h, s_wtot, s_out, &T, &last);
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) {
    const uint32_t n = t + (uint32_t)j * kFinishThreads;
    if (n < n_all) {
      const uint32_t k = keys[j];
      mrow[n] = (n < vn32 && (k > T || (k == T && n <= last))) ? 1 : 0;
    }
  }
}

// Subset top-K of short lists (as short rows above) in one launch instead
// of subset scan + finish: one block per row gathers the keys of its list
// positions into registers (thread t holds positions kShortPer t onwards,
// so the chosen ones leave in list order after one block scan), selects
// exactly over the positions with a key (an index in [0, N)) and writes the
// chosen chunk indices and their number.  Ties go to the earlier position,
// as on the other paths.
template <int kShortPer>
__global__ __launch_bounds__(kFinishThreads) void subset_short_kernel(const float* __restrict__ scores, int64_t N,
                                                                      const int32_t* __restrict__ subset,
                                                                      const int32_t* __restrict__ n_subset,
                                                                      int32_t cap, int32_t top_k,
                                                                      int32_t* __restrict__ out,
                                                                      int32_t* __restrict__ n_out) {
  __shared__ __attribute__((aligned(16))) uint32_t h[2 * kSelBins];
  __shared__ uint32_t s_wtot[kFinishThreads / 64];
  __shared__ uint32_t s_out[3];
  const int b = blockIdx.x;
  const uint32_t t = threadIdx.x;
  const int64_t n64 = n_subset ? (int64_t)n_subset[b] : (int64_t)cap;
  const uint32_t n = (uint32_t)(n64 < 0 ? 0 : (n64 > cap ? cap : n64));  // cap <= kShortPer kFinishThreads
  if (top_k == 0 || n == 0) {  // uniform over the block
    if (t == 0) n_out[b] = 0;
    return;
  }
  const int32_t* srow = subset + (size_t)b * cap;
  const float* row = scores + (size_t)b * N;
  const uint32_t p0 = t * kShortPer;
  int32_t idx[kShortPer];
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) idx[j] = p0 + j < n ? srow[p0 + j] : -1;
  uint32_t keys[kShortPer];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) {
    const bool ok = idx[j] >= 0 && (int64_t)idx[j] < N;
    keys[j] = ok ? order_key(row[idx[j]]) : 0u;
    mine += keys[j] != 0u ? 1u : 0u;
  }
  uint32_t n_keyed;
  (void)block_excl_scan(mine, s_wtot, &n_keyed);
  uint32_t K = (uint32_t)top_k;
  uint32_t T = 0u, last = 0xffffffffu;
  const bool all = K >= n_keyed;  // uniform
  if (all) {
    K = n_keyed;
  } else {
    auto each = [&](auto f) {
#pragma unroll
      for (int j = 0; j < kShortPer; ++j)
        if (keys[j] != 0u) f(make_uint2(keys[j], p0 + j));
    };
    radix_select<kFinishThreads>(each, K, index_bits(n), h, s_wtot, s_out, &T, &last);
  }
  uint32_t chosen = 0u, cnt = 0u;
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) {
    const uint32_t k = keys[j];
    const bool c = k != 0u && (all || k > T || (k == T && p0 + j <= last));
    chosen |= (c ? 1u : 0u) << j;
    cnt += c ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t pos = block_excl_scan(cnt, s_wtot, &tot);
  int32_t* orow = out + (size_t)b * top_k;
#pragma unroll
  for (int j = 0; j < kShortPer; ++j)
    if ((chosen >> j) & 1u) {
      if (pos < (uint32_t)top_k) orow[pos] = idx[j];
      ++pos;
    }
  if (t == 0) n_out[b] = (int32_t)K;
}

// Threshold mask: 16 chunks per thread, one 16-byte store when the run is
// whole and aligned.  grid = (ceil(N / kScanSlice), B), block = kScanThreads.
__global__ __launch_bounds__(kScanThreads) void threshold_kernel(const float* __restrict__ scores, int64_t N,
                                                                 const int32_t* __restrict__ valid_n,
                                                                 float threshold, uint8_t* __restrict__ mask) {
  const int b = blockIdx.y;
  const int64_t vn = row_valid(valid_n, b, N);
  const int64_t n0 = ((int64_t)blockIdx.x * kScanThreads + threadIdx.x) * kSub;
  if (n0 >= N) return;
  const float* row = scores + (size_t)b * N;
  uint8_t* mrow = mask + (size_t)b * N;
  if (n0 + kSub <= vn && ((((uintptr_t)(row + n0)) & 15) == 0) && ((((uintptr_t)(mrow + n0)) & 15) == 0)) {
    float4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *(const float4*)(row + n0 + 4 * q);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (v[q].x > threshold ? 1u : 0u) | (v[q].y > threshold ? 0x100u : 0u) |
             (v[q].z > threshold ? 0x10000u : 0u) | (v[q].w > threshold ? 0x1000000u : 0u);
    *(uint4*)(mrow + n0) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    for (int j = 0; j < kSub && n0 + j < N; ++j) mrow[n0 + j] = (n0 + j < vn && row[n0 + j] > threshold) ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_select_topk(const Workspace& ws, const float* scores, int B, int64_t N, const int32_t* valid_n,
                              int32_t top_k, uint8_t* mask, hipStream_t stream) {
  const int per = short_per(N, top_k);
  if (per != 0) {
    auto kern = per == (int)(kShortRow / kFinishThreads) ? topk_short_kernel<(int)(kShortRow / kFinishThreads)>
                                                         : topk_short_kernel<(int)(kShortRowMax / kFinishThreads)>;
    hipLaunchKernelGGL(kern, dim3(B), dim3(kFinishThreads), 0, stream, scores, N, valid_n, top_k, mask);
    return hipGetLastError();
  }
  const unsigned slices = (unsigned)((N + kScanSlice - 1) / kScanSlice);
  hipLaunchKernelGGL(topk_scan_kernel, dim3(slices, B), dim3(kScanThreads), 0, stream, scores, N, valid_n, top_k,
                     ws.tile_info, mask);
  hipLaunchKernelGGL(topk_finish_kernel<false>, dim3(B), dim3(kFinishThreads), 0, stream, scores, N, valid_n, top_k,
                     (const uint2*)ws.tile_info, mask, (const uint32_t*)nullptr, (const int32_t*)nullptr,
                     (const int32_t*)nullptr, 0, (int32_t*)nullptr, (int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_select_topk_subset_fast(const Workspace& ws, const float* scores, int B, int64_t N,
                                          const int32_t* subset, const int32_t* n_subset, int32_t cap, int32_t top_k,
                                          int32_t* out, int32_t* n_out, hipStream_t stream) {
  const int per = short_per(cap, top_k);
  if (per != 0) {
    auto kern = per == (int)(kShortRow / kFinishThreads) ? subset_short_kernel<(int)(kShortRow / kFinishThreads)>
                                                         : subset_short_kernel<(int)(kShortRowMax / kFinishThreads)>;
    hipLaunchKernelGGL(kern, dim3(B), dim3(kFinishThreads), 0, stream, scores, N, subset, n_subset, cap, top_k, out,
                       n_out);
    return hipGetLastError();
  }
  const unsigned slices = (unsigned)((cap + kSubScanSlice - 1) / kSubScanSlice);
  if (slices > 0)
    hipLaunchKernelGGL(subset_scan_kernel, dim3(slices, B), dim3(kScanThreads), 0, stream, scores, N, subset, n_subset,
                       cap, top_k, ws.sub_keys, ws.sub_tiles);
  hipLaunchKernelGGL(topk_finish_kernel<true>, dim3(B), dim3(kFinishThreads), 0, stream, scores, N,
                     (const int32_t*)nullptr, top_k, (const uint2*)ws.sub_tiles, (uint8_t*)nullptr,
                     (const uint32_t*)ws.sub_keys, subset, n_subset, cap, out, n_out);
  return hipGetLastError();
}

hipError_t launch_select_threshold(const float* scores, int B, int64_t N, const int32_t* valid_n, float threshold,
                                   uint8_t* mask, hipStream_t stream) {
  const unsigned slices = (unsigned)((N + kScanSlice - 1) / kScanSlice);
  hipLaunchKernelGGL(threshold_kernel, dim3(slices, B), dim3(kScanThreads), 0, stream, scores, N, valid_n, threshold,
                     mask);
  return hipGetLastError();
}

}  // namespace fm
