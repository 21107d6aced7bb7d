// Per-layer chunk score and ensemble (FlashMemory DS-V4 Retriever README,
// "compressed_k format", "Architecture" score line, "Joint checkpoint +
// ensemble"):
//   k       = e4m3(bytes[0:128]) * f32le(bytes[128:132])
//   S_l     = sigmoid( sum_h relu(k . q_{l,h}) * w_{l,h} ),  l = l10, l12, l20
//   E       = max_l S_l  or  mean_l S_l
//
// Per request row this is a [N x 128] x [128 x 192] contraction (3 layers x
// 64 heads), 49152 flop per 132-byte chunk, on the 16x16x32 f16 MFMA
// (plus 4096 flop per chunk for the linear term below).
//
// Exact-algebra choices that keep it within the fp64 result:
//   - the e4m3 codes are converted exactly to f16 (every finite e4m3 value
//     is an f16 value) and the fp32 scale s multiplies fp32 head sums
//     instead of the operand;
//   - q is rounded once to f16 (11-bit significand);
//   - relu(y) = (y + |y|) / 2.  With x_h = code . q_h (q_h in f16) and
//     y_h = s x_h:
//       sum_h w_h relu(y_h) = s/2 * sum_h w_h x_h + |s|/2 * sum_h w_h |x_h|.
//     The first sum is linear in the codes: it is (sum_h w_h q_h) . code,
//     four more MFMAs per tile on spare A rows holding the weighted query
//     sum of each layer split into two f16 parts (hi + lo, about 22
//     significant bits).  The second is one fused multiply-add per head with
//     an absolute-value operand, and a scale of either sign costs nothing;
//   - max ensemble: max_l sigmoid(t_l) = sigmoid(max_l t_l), one sigmoid.
#include <algorithm>

#include "fm_score_common.h"

namespace fm {
namespace {

using namespace score;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// MFMA 16x16x32 f16 operand layout: lane l supplies A[l%16][8(l/16) + e] and
// B[8(l/16) + e][l%16], e = 0..7, and receives C[4(l/16) + r][l%16].
// A = queries (rows = 16 heads of a head tile), B = keys (columns = 16
// chunks).  For k-step t (t = 0..3) lane l's eight k slots are the dims
// 32(l/16) + 8t + e, so each lane reads one contiguous 32-byte run of its
// chunk's codes.  Fragment f = (layer * 4 + head_tile) * 4 + t for the
// heads; fragment 48 + t holds the linear-term rows for k-step t: row l
// (l < 3) is the high f16 part of v_l = 1/2 sum_h w_{l,h} q_{l,h} (with q
// already rounded to f16, the sum in fp32), row 4 + l the low part
// v_l - hi, other rows zero.  The MFMA output of that tile then holds, in
// lane group 0, the high part of layer r's term in element r, and in lane
// group 1 the low part.
// One block per (row, layer), 256 threads.  Thread t packs the head
// fragments o = t + 256 j (j = 0..3; fragment o / 64, lane o % 64) from two
// float4 loads each, all issued first, and keeps the f16 queries in LDS;
// then v_d = 1/2 sum_h w_h q_hd is summed in two head halves (fp32), split
// into hi + lo f16 parts and scattered to the linear-term rows of this
// layer.  The layer-0 block also writes the zero rows.
__global__ __launch_bounds__(256) void pack_q_kernel(const float* __restrict__ q, const float* __restrict__ w, int B,
                                                     f16x8* __restrict__ qpack) {
  __shared__ __attribute__((aligned(16))) _Float16 qs[kHeads][kHeadDim + 8];
  __shared__ float red[2][kHeadDim];
  __shared__ __attribute__((aligned(16))) _Float16 lin[4][4][2][8];  // [t][g][hi, lo][e]
  const int b = blockIdx.x / kLayers;
  const int layer = blockIdx.x % kLayers;
  const int t = threadIdx.x;
  const float* qb = q + ((size_t)layer * B + b) * kHeads * kHeadDim;
  f16x8* out = qpack + (size_t)b * kQFrags * 64;
  float4 v[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = t + 256 * j;
    const int f = o >> 6, lane = o & 63;
    const int head = 16 * (f >> 2) + (lane & 15);
    const int d0 = 32 * (lane >> 4) + 8 * (f & 3);
    v[j][0] = *(const float4*)(qb + head * kHeadDim + d0);
    v[j][1] = *(const float4*)(qb + head * kHeadDim + d0 + 4);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = t + 256 * j;
    const int f = o >> 6, lane = o & 63;
    const int head = 16 * (f >> 2) + (lane & 15);
    const int d0 = 32 * (lane >> 4) + 8 * (f & 3);
    const f16x8 h = {(_Float16)v[j][0].x, (_Float16)v[j][0].y, (_Float16)v[j][0].z, (_Float16)v[j][0].w,
                     (_Float16)v[j][1].x, (_Float16)v[j][1].y, (_Float16)v[j][1].z, (_Float16)v[j][1].w};
    out[(layer * 16 + f) * 64 + lane] = h;
    *(f16x8*)&qs[head][d0] = h;
  }
  __syncthreads();
  {
    const int d = t & (kHeadDim - 1), half = t >> 7;
    const float* wb = w + ((size_t)layer * B + b) * kHeads + 32 * half;
    float acc = 0.f;
#pragma unroll 8
    for (int h = 0; h < 32; ++h) acc = fmaf(wb[h], (float)qs[32 * half + h][d], acc);
    red[half][d] = acc;
  }
  __syncthreads();
  if (t < kHeadDim) {
    const float vd = 0.5f * (red[0][t] + red[1][t]);
    const _Float16 hi = (_Float16)vd;
    const _Float16 lo = (_Float16)(vd - (float)hi);
    const int g = t >> 5, ks = (t >> 3) & 3, e = t & 7;  // dim t = 32 g + 8 ks + e
    lin[ks][g][0][e] = hi;
    lin[ks][g][1][e] = lo;
  }
  __syncthreads();
  if (t < 32) {
    const int ks = t >> 3, g = (t >> 1) & 3, part = t & 1;
    const int row = part ? 4 + layer : layer;
    out[(kQHeadFrags + ks) * 64 + row + 16 * g] = *(const f16x8*)&lin[ks][g][part][0];
  }
  if (layer == 0 && t < 4 * 4 * 10) {  // rows 3, 7, 8 .. 15 of every (k-step, lane group)
    const int ks = t / 40, g = (t / 10) & 3, z = t % 10;
    const int row = z == 0 ? 3 : (z == 1 ? 7 : 6 + z);
    out[(kQHeadFrags + ks) * 64 + row + 16 * g] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

__device__ __forceinline__ f16x8 decode8(uint32_t lo, uint32_t hi) {
  // four 2-code conversions; scale 1.0 leaves the value unchanged
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ void decode_tile(const RawTile& t, f16x8 (&kf)[4]) {
  kf[0] = decode8(t.lo[0], t.lo[1]);
  kf[1] = decode8(t.lo[2], t.lo[3]);
  kf[2] = decode8(t.hi[0], t.hi[1]);
  kf[3] = decode8(t.hi[2], t.hi[3]);
}

__device__ __forceinline__ void mfma_tile(const f16x8 (&qf)[kLayers][4][4], const f16x8 (&ql)[4], const f16x8 (&kf)[4],
                                          f32x4 (&acc)[kLayers][4], f32x4& lin) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[l][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[l][mt][0], kf[0], zero, 0, 0, 0);
  lin = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[0], kf[0], zero, 0, 0, 0);
#pragma unroll
  for (int t = 1; t < 4; ++t) {
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[l][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[l][mt][t], kf[t], acc[l][mt], 0, 0, 0);
    lin = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[t], kf[t], lin, 0, 0, 0);
  }
}

// Head reduction, sigmoid, ensemble and store of one tile.  wh = w / 2.
template <bool MEAN, bool PER_LAYER>
__device__ __forceinline__ void finish_tile(const Ctx& cx, const f32x4 (&acc)[kLayers][4], const f32x4& lin,
                                            const f32x4 (&wh)[kLayers][4], float s, int tile) {
  float t[kLayers];
#pragma unroll
  for (int l = 0; l < kLayers; ++l) {
    float p = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) p = fmaf(fabsf(acc[l][mt][r]), wh[l][mt][r], p);
    // |s| p + s lin: lane group 0 adds the high part of the linear term,
    // group 1 the low part, groups 2 and 3 hold zeros there.
    t[l] = sum4groups(fmaf(s, lin[l], fabsf(s) * p));  // the layer's logit
  }
  store_tile<MEAN, PER_LAYER>(cx, t, tile);
}

// Instruction order of one phase for the scheduler: every MFMA followed by
// two vector-ALU instructions (a wave issues in order, so the vector work
// of the reduction and decode must sit between the MFMAs to overlap them),
// then the phase's requests (after the decode has consumed the ring slot
// they refill) and its stores.
__device__ __forceinline__ void interleave_phase() {
#pragma unroll
  for (int k = 0; k < kLayers * 4 * 4 + 4; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);    // VMEM read: codes, scale
  __builtin_amdgcn_sched_group_barrier(0x040, 4, 0);    // VMEM write
  // Nothing crosses a phase boundary: the scheduler would otherwise sink a
  // request next to the decode that consumes it, phases later.
  __builtin_amdgcn_sched_barrier(0);
}

// One pipeline run: tiles of chunks [start, start + count) of row b, every
// chunk below the row's valid_n.
//
// Software pipeline, one wave per SIMD: in the phase of tile i the wave
// issues the 52 MFMAs of tile i, interleaved with the reduction of tile i-1
// and the decode of tile i+1; the records of tile i+6 are requested in the
// same phase (6 tiles in flight).  Tiles past the run's chunks read as zeros
// and their stores are dropped by the buffer range checks.
template <bool MEAN, bool PER_LAYER>
__device__ __forceinline__ void score_run(const f16x8* __restrict__ qpack, const float* __restrict__ w,
                                          const uint8_t* __restrict__ comp_k, int B, int64_t N, int b, int64_t start,
                                          int64_t count, int lane, float* __restrict__ scores,
                                          float* __restrict__ per_layer) {
  const Ctx cx = make_ctx<PER_LAYER>(comp_k, B, N, b, start, count, lane, scores, per_layer);

  // Query fragments, linear-term fragments and w: every load is issued
  // before the first use, so the wave pays one memory latency here, not one
  // per fragment.
  f16x8 qf[kLayers][4][4];
  f16x8 ql[4];
  f32x4 wv[kLayers][4];  // w / 2 of the heads this lane's accumulators hold: 16 mt + 4 g + r
  {
    const f16x8* qp = qpack + (size_t)b * kQFrags * 64 + lane;
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) qf[l][mt][t] = qp[((l * 4 + mt) * 4 + t) * 64];
#pragma unroll
    for (int t = 0; t < 4; ++t) ql[t] = qp[(kQHeadFrags + t) * 64];
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) wv[l][mt] = *(const f32x4*)(w + ((size_t)l * B + b) * kHeads + 16 * mt + 4 * cx.g);
  }
  // The first records are requested after the queries and weights, one tile
  // at a time in tile order: the waits before the loop then cover only the
  // queries and weights, and those in the loop count record loads alone.
  __builtin_amdgcn_sched_barrier(0);
  RawTile ring[kRing];
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    load_tile(cx, k, ring[k]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Keep the query fragments in accumulation registers: the MFMA reads its A
  // operand from there, leaving the vector registers to the accumulators,
  // decoded keys and records in flight.
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) asm volatile("" : "+a"(qf[l][mt][t]));
#pragma unroll
  for (int t = 0; t < 4; ++t) asm volatile("" : "+a"(ql[t]));
  // Consume w here, so its wait is paid before the loop; a wait inside the
  // loop would also drain the records in flight.
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      wv[l][mt] = 0.5f * wv[l][mt];
      asm volatile("" : "+v"(wv[l][mt]));
    }

  const int tiles = (int)((count + kTile - 1) / kTile);

  f16x8 kf[2][4];
  f32x4 acc[2][kLayers][4];
  f32x4 lin[2];

  // Phase of tile i, P = i mod 8 (compile-time, so every register index is
  // static): MFMAs of tile i; finish tile i-1 (its scale still in its ring
  // slot); decode tile i+1 (requested five phases ago); request tile i+6
  // into the slot of tile i-2, finished in the previous phase.
#define FM_PHASE(P, I)                                                                                \
  {                                                                                                   \
    mfma_tile(qf, ql, kf[(P) & 1], acc[(P) & 1], lin[(P) & 1]);                                       \
    finish_tile<MEAN, PER_LAYER>(cx, acc[((P) + 1) & 1], lin[((P) + 1) & 1], wv, ring[((P) + 7) & 7].s,  \
                                 (I) - 1);                                                            \
    decode_tile(ring[((P) + 1) & 7], kf[((P) + 1) & 1]);                                              \
    load_tile(cx, (I) + kAhead, ring[((P) + 6) & 7]);                                                 \
    interleave_phase();                                                                               \
  }

  // Tile 0 (nothing to finish yet).
  decode_tile(ring[0], kf[0]);
  mfma_tile(qf, ql, kf[0], acc[0], lin[0]);
  decode_tile(ring[1], kf[1]);
  load_tile(cx, kAhead, ring[kAhead]);

  // Tiles 1 .. 8 m, eight per iteration, branch-free.  Tiles past the last
  // valid one read zeros and their stores are dropped, so the count can be
  // rounded up; a full wave has 8 m + 1 tiles and wastes none.
  int i = 1;
  do {
    FM_PHASE(1, i)
    FM_PHASE(2, i + 1)
    FM_PHASE(3, i + 2)
    FM_PHASE(4, i + 3)
    FM_PHASE(5, i + 4)
    FM_PHASE(6, i + 5)
    FM_PHASE(7, i + 6)
    FM_PHASE(0, i + 7)
    i += 8;
  } while (i < tiles);
  finish_tile<MEAN, PER_LAYER>(cx, acc[0], lin[0], wv, ring[0].s, i - 1);  // tile i - 1 = 0 mod 8
#undef FM_PHASE
}

// grid = number of compute units, block = 256 (one wave per SIMD); each wave
// scores its share of the tile list (walk_share).
template <bool MEAN, bool PER_LAYER>
__global__ __launch_bounds__(256, 1) void score_kernel(const f16x8* __restrict__ qpack, const float* __restrict__ w,
                                                       const uint8_t* __restrict__ comp_k, int B, int64_t N,
                                                       const int32_t* __restrict__ valid_n,
                                                       const int64_t* __restrict__ row_tiles,
                                                       const int32_t* __restrict__ wave_row,
                                                       int64_t total_tiles,  // used when row_tiles is null
                                                       float* __restrict__ scores, float* __restrict__ per_layer) {
  const int lane = threadIdx.x & 63;
  walk_share(B, N, valid_n, row_tiles, wave_row, total_tiles, [&](int b, int64_t start, int64_t count) {
    score_run<MEAN, PER_LAYER>(qpack, w, comp_k, B, N, b, start, count, lane, scores, per_layer);
  });
}

// Plan for ragged rows (one block of 1024 threads): row_tiles[b] = sum of
// ceil(valid_n / 16) over the rows before b (row_tiles[B] = all tiles), and
// for each wave the row holding its first tile.
__global__ __launch_bounds__(1024) void score_plan_kernel(const int32_t* __restrict__ valid_n, int B, int64_t N,
                                                          int waves, int64_t* __restrict__ row_tiles,
                                                          int32_t* __restrict__ wave_row) {
  __shared__ int64_t s_pre[4096 + 1];
  __shared__ int64_t s_wsum[16];
  const int t = threadIdx.x;
  const int per = (B + 1023) / 1024;  // rows per thread, consecutive
  int64_t cnt[4] = {0, 0, 0, 0};
  int64_t tot = 0;
  for (int j = 0; j < per; ++j) {
    const int r = t * per + j;
    if (r < B) {
      const int64_t v = valid_n[r];
      const int64_t vn = v < 0 ? 0 : (v > N ? N : v);
      cnt[j] = (vn + kTile - 1) / kTile;
      tot += cnt[j];
    }
  }
  // Exclusive scan of the per-thread totals: wave shuffles, then across waves.
  int64_t incl = tot;
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(incl, off, 64);
    if ((t & 63) >= off) incl += v;
  }
  if ((t & 63) == 63) s_wsum[t >> 6] = incl;
  __syncthreads();
  int64_t before = 0;
  for (int wv = 0; wv < (t >> 6); ++wv) before += s_wsum[wv];
  int64_t acc = before + incl - tot;
  for (int j = 0; j < per; ++j) {
    const int r = t * per + j;
    if (r < B) {
      s_pre[r] = acc;
      acc += cnt[j];
    }
  }
  if (t == 1023) s_pre[B] = before + incl;  // the last thread's inclusive total is the grand total
  __syncthreads();
  const int64_t total = s_pre[B];
  for (int r = t; r <= B; r += 1024) row_tiles[r] = s_pre[r];
  for (int g = t; g < waves; g += 1024) {
    const int64_t first = (int64_t)g * total / waves;
    int lo = 0, hi = B - 1;  // largest row with s_pre[row] <= first
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= first) lo = mid;
      else hi = mid - 1;
    }
    wave_row[g] = lo;
  }
}

// -inf for the chunks of each row at or beyond its valid_n.
template <bool PER_LAYER>
__global__ __launch_bounds__(256) void score_tail_kernel(const int32_t* __restrict__ valid_n, int B, int64_t N,
                                                         float* __restrict__ scores, float* __restrict__ per_layer) {
  const int b = blockIdx.y;
  const int64_t v = valid_n[b];
  const int64_t vn = v < 0 ? 0 : (v > N ? N : v);
  const float ninf = -__builtin_huge_valf();
  for (int64_t n = vn + (int64_t)blockIdx.x * 256 + threadIdx.x; n < N; n += (int64_t)gridDim.x * 256) {
    scores[(size_t)b * N + n] = ninf;
    if (PER_LAYER)
      for (int l = 0; l < kLayers; ++l) per_layer[((size_t)l * B + b) * N + n] = ninf;
  }
}

}  // namespace

hipError_t launch_score_plan(const Workspace& ws, const int32_t* valid_n, int B, int64_t N, float* scores,
                             float* per_layer, hipStream_t stream, const int64_t** row_tiles, int64_t* total_tiles) {
  *total_tiles = (int64_t)B * ((N + kTile - 1) / kTile);
  *row_tiles = nullptr;
  if (valid_n) {
    hipLaunchKernelGGL(score_plan_kernel, dim3(1), dim3(1024), 0, stream, valid_n, B, N, 4 * ws.score_blocks,
                       ws.row_tiles, ws.wave_row);
    *row_tiles = ws.row_tiles;
    const unsigned gx = (unsigned)std::min<int64_t>((N + 255) / 256, 64);
    if (per_layer)
      hipLaunchKernelGGL(score_tail_kernel<true>, dim3(gx, B), dim3(256), 0, stream, valid_n, B, N, scores, per_layer);
    else
      hipLaunchKernelGGL(score_tail_kernel<false>, dim3(gx, B), dim3(256), 0, stream, valid_n, B, N, scores, per_layer);
  }
  return hipGetLastError();
}

hipError_t launch_score(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B, int64_t N,
                        const int32_t* valid_n, int mode, float* scores, float* per_layer, hipStream_t stream) {
  f16x8* qpack = (f16x8*)ws.qpack;
  hipLaunchKernelGGL(pack_q_kernel, dim3(B * kLayers), dim3(256), 0, stream, q, w, B, qpack);
  const int64_t* row_tiles;
  int64_t total_tiles;
  hipError_t e = launch_score_plan(ws, valid_n, B, N, scores, per_layer, stream, &row_tiles, &total_tiles);
  if (e != hipSuccess) return e;
  const bool mean = mode == FM_ENSEMBLE_MEAN;
  auto kern = mean ? (per_layer ? score_kernel<true, true> : score_kernel<true, false>)
                   : (per_layer ? score_kernel<false, true> : score_kernel<false, false>);
  hipLaunchKernelGGL(kern, dim3(ws.score_blocks), dim3(256), 0, stream, (const f16x8*)qpack, w, comp_k, B, N, valid_n,
                     row_tiles, (const int32_t*)ws.wave_row, total_tiles, scores, per_layer);
  return hipGetLastError();
}

}  // namespace fm
