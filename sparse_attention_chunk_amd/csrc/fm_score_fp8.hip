// Per-layer chunk score and ensemble on the fp8 matrix cores: the same
// definition as fm_score.hip (FlashMemory DS-V4 Retriever README,
// "compressed_k format", "Architecture" score line, "Joint checkpoint +
// ensemble"), in the native-FP8 indexer form that the same README's "Is /
// is not" section names for production.
//
// The e4m3 codes of the records enter the 16x16x128 fp8 MFMA as stored (no
// decode); the queries are split into two e4m3 parts:
//   - per (row, layer, head) the query is scaled by 2^a (a power of two
//     putting its largest |element| in [128, 256)), then hi = e4m3(q 2^a)
//     and lo = e4m3(q 2^a - hi).  hi + lo carries about 8 significant bits
//     (relative error at most 2^-8 of an element, plus the e4m3 subnormal
//     floor 2^-10 at scale 2^a); one MFMA per part, the same accumulator;
//   - the head weight w/2 absorbs 2^-a (exact power-of-two scaling);
//   - relu(y) = (y + |y|) / 2 as in the f16 path: the linear term uses
//     v_l = 1/2 sum_h w_h (hi + lo) 2^-a, scaled by 2^b_l and split into
//     three e4m3 parts on rows l, 4 + l and 8 + l of one more fragment, so
//     lane groups 0..2 of that MFMA's output hold the three parts of layer
//     l's term in element l; the logit takes them times s 2^-b_l.
// Per 16-chunk tile: 24 MFMAs for the heads (3 layers x 4 head tiles x 2
// parts) + 1 for the linear terms, 32 cycles each (the f16 path: 52 x 16).
// Measured on the synthetic workloads the scores stay within 6e-4 of the
// fp64 result (the f16 path: 2.3e-4).
#include <algorithm>

#include "fm_score_common.h"

namespace fm {
namespace {

using namespace score;

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// MFMA 16x16x128 fp8 operand layout: lane l supplies A[l%16][32(l/16) + e]
// and B[32(l/16) + e][l%16], e = 0..31 (32 bytes), and receives
// C[4(l/16) + r][l%16].  A = query parts (rows = 16 heads of a head tile),
// B = codes (columns = 16 chunks): lane l's B bytes are one contiguous
// 32-byte run of its chunk's codes, the same run the f16 path loads.
// Fragment f = (layer * 4 + head_tile) * 2 + part holds the hi (part 0) or
// lo (part 1) query bytes; fragment 24 the linear-term rows.
__device__ __forceinline__ f32x4 mfma8(const i32x8& a, const i32x8& b, const f32x4& c) {
  // Format codes 0 (e4m3) for both operands; no block scales.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// The linear term: A block scales sa (E8M0 code per row and 32-wide block,
// supplied by the lane holding the block; 127 is 1), B unscaled.
__device__ __forceinline__ f32x4 mfma8_scaled(const i32x8& a, int32_t sa, const i32x8& b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, sa, 0, 127);
}

// Four floats -> four e4m3 bytes (round to nearest even), and back.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

__device__ __forceinline__ void e4m3x4_value(uint32_t v, float (&f)[4]) {
  f[0] = __builtin_amdgcn_cvt_f32_fp8((int)v, 0);
  f[1] = __builtin_amdgcn_cvt_f32_fp8((int)v, 1);
  f[2] = __builtin_amdgcn_cvt_f32_fp8((int)v, 2);
  f[3] = __builtin_amdgcn_cvt_f32_fp8((int)v, 3);
}

// 2^a with m 2^a in [128, 256) (m > 0); 0 for m = 0.
__device__ __forceinline__ int part_exponent(float m) {
  if (!(m > 0.f)) return 0;
  int ex;
  (void)frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
  return 8 - ex;
}

// One block per (row, layer), 256 threads: thread t owns head t / 4, dims
// 32 (t % 4) .. + 31, i.e. lane (head % 16) + 16 (t % 4) of the head tile's
// two fragments.  Writes the hi and lo fragments, the scaled half weights
// w8[row][layer 64 + h] = w_h 2^-a_h / 2, then the linear-term rows of this
// layer and their block-scale codes 127 - b (2^-b) at w8[row][192 + lane].
// The layer-0 block also writes the zero rows of the linear-term fragment
// and their codes (127).
__global__ __launch_bounds__(256) void pack_q8_kernel(const float* __restrict__ q, const float* __restrict__ w, int B,
                                                      uint4* __restrict__ qpack8, float* __restrict__ w8) {
  __shared__ float qs[kHeads][kHeadDim + 4];  // the dequantised query hi + lo
  __shared__ float red[2][kHeadDim];
  __shared__ float wmax[2];
  __shared__ __attribute__((aligned(16))) uint32_t lin8[3][kHeadDim / 4];  // [part][dims / 4]
  __shared__ float w_s[kHeads];  // the row's head weights, loaded with q (not in the sum's loop)
  const int b = blockIdx.x / kLayers;
  const int layer = blockIdx.x % kLayers;
  const int t = threadIdx.x;
  const int h = t >> 2, g = t & 3;
  const float* qh = q + (((size_t)layer * B + b) * kHeads + h) * kHeadDim + 32 * g;
  const float wh = w[((size_t)layer * B + b) * kHeads + h];
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 x = *(const float4*)(qh + 4 * i);
    v[4 * i] = x.x;
    v[4 * i + 1] = x.y;
    v[4 * i + 2] = x.z;
    v[4 * i + 3] = x.w;
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1));  // the head's four threads are lanes 4k .. 4k + 3
  m = fmaxf(m, __shfl_xor(m, 2));
  const int a = part_exponent(m);
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float r[4], hv[4], lr[4], lv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = ldexpf(v[4 * i + j], a);
    hi[i] = e4m3x4(r[0], r[1], r[2], r[3]);
    e4m3x4_value(hi[i], hv);
#pragma unroll
    for (int j = 0; j < 4; ++j) lr[j] = r[j] - hv[j];  // exact: hv is r rounded to 4 significant bits
    lo[i] = e4m3x4(lr[0], lr[1], lr[2], lr[3]);
    e4m3x4_value(lo[i], lv);
#pragma unroll
    for (int j = 0; j < 4; ++j) qs[h][32 * g + 4 * i + j] = ldexpf(hv[j] + lv[j], -a);
  }
  {
    const int f = (layer * 4 + (h >> 4)) * 2;
    const int lane = (h & 15) + 16 * g;
    uint4* out = qpack8 + ((size_t)b * kQ8Frags * 64 + (size_t)f * 64 + lane) * 2;
    out[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    out[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    out += 64 * 2;  // fragment f + 1
    out[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    out[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
  }
  if (g == 0) {
    w8[(size_t)b * kW8Row + layer * kHeads + h] = ldexpf(0.5f * wh, -a);
    w_s[h] = wh;
  }
  __syncthreads();

  // v_d = 1/2 sum_h w_h q_hd over the dequantised parts, in two head halves.
  {
    const int d = t & (kHeadDim - 1), half = t >> 7;
    float acc = 0.f;
#pragma unroll 8
    for (int k = 0; k < 32; ++k) acc = fmaf(w_s[32 * half + k], qs[32 * half + k][d], acc);
    red[half][d] = acc;
  }
  __syncthreads();
  float u = 0.f;
  if (t < kHeadDim) {
    u = 0.5f * (red[0][t] + red[1][t]);
    float mu = fabsf(u);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mu = fmaxf(mu, __shfl_xor(mu, off));
    if ((t & 63) == 0) wmax[t >> 6] = mu;
  }
  __syncthreads();
  if (t < kHeadDim) {
    const int bl = part_exponent(fmaxf(wmax[0], wmax[1]));
    float r = ldexpf(u, bl);
    uint32_t p[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      p[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.f, 0, false) & 0xffu;
      r -= __builtin_amdgcn_cvt_f32_fp8((int)p[k], 0);
    }
    // Gather the bytes of four consecutive dims into one word (lanes t..t+3).
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      uint32_t word = p[k] << (8 * (t & 3));
      word |= __shfl_xor(word, 1);
      word |= __shfl_xor(word, 2);
      if ((t & 3) == 0) lin8[k][t >> 2] = word;
    }
    // Block-scale codes of this layer's rows (4k + layer, k = 0..2; 2^-b
    // below 2^-127 clamped to 2^-127), code 127 for the zero rows (layer 0).
    const int r16 = t & 15;
    const bool mine = r16 < 12 && (r16 & 3) == layer;
    const bool zero_row = r16 >= 12 || (r16 & 3) == 3;
    const int code = 127 - bl < 0 ? 0 : (127 - bl > 254 ? 254 : 127 - bl);
    if (t < 64 && (mine || (layer == 0 && zero_row)))
      ((int32_t*)(w8 + (size_t)b * kW8Row + kLayers * kHeads))[t] = mine ? code : 127;
  }
  __syncthreads();
  uint4* lin_out = qpack8 + ((size_t)b * kQ8Frags * 64 + (size_t)kQ8HeadFrags * 64) * 2;
  if (t < 12) {  // part k = t / 4 of this layer, dims 32 j .. + 31 with j = t % 4
    const int k = t >> 2, j = t & 3;
    const int lane = 4 * k + layer + 16 * j;
    const uint4* src = (const uint4*)&lin8[k][8 * j];
    lin_out[2 * lane] = src[0];
    lin_out[2 * lane + 1] = src[1];
  }
  if (layer == 0 && t >= 16 && t < 16 + 28) {  // rows 3, 7, 11 .. 15 of every lane group
    const int z = (t - 16) >> 2, j = (t - 16) & 3;
    const int row = z < 3 ? 4 * z + 3 : 9 + z;
    const int lane = row + 16 * j;
    lin_out[2 * lane] = make_uint4(0, 0, 0, 0);
    lin_out[2 * lane + 1] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ i32x8 tile_codes(const RawTile& t) {
  return i32x8{(int)t.lo[0], (int)t.lo[1], (int)t.lo[2], (int)t.lo[3],
               (int)t.hi[0], (int)t.hi[1], (int)t.hi[2], (int)t.hi[3]};
}

// The 25 MFMAs of one tile: the hi parts of every head tile first, then the
// linear term, then the lo parts, so no MFMA waits on the one before it.
__device__ __forceinline__ void mfma_tile8(const i32x8 (&qh)[kLayers][4], const i32x8 (&ql)[kLayers][4],
                                           const i32x8& qlin, int32_t qsc, const i32x8& k, f32x4 (&acc)[kLayers][4],
                                           f32x4& lin) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[l][mt] = mfma8(qh[l][mt], k, zero);
  lin = mfma8_scaled(qlin, qsc, k);
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[l][mt] = mfma8(ql[l][mt], k, acc[l][mt]);
}

// Head reduction, sigmoid, ensemble and store of one tile, in the phase
// P = (tile + 1) mod 8.  wv = w 2^-a / 2 of this lane's heads; lin is
// already times 2^-b_l (the MFMA's block scales).  Scores only: in four-tile groups, as in the f16 kernel (the
// phases P = 4 and 0 reduce and store the group); with per-layer scores,
// every tile on its own.
template <bool MEAN, bool PER_LAYER, int P>
__device__ __forceinline__ void finish_tile8(const Ctx& cx, const f32x4 (&acc)[kLayers][4], const f32x4& lin,
                                             const f32x4 (&wv)[kLayers][4], float s, int tile, float (&x)[4]) {
  float t[kLayers];
  const float sg = __builtin_copysignf(1.0f, s);
#pragma unroll
  for (int l = 0; l < kLayers; ++l) {
    float p = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) p = fmaf(fabsf(acc[l][mt][r]), wv[l][mt][r], p);
    // (s 2^-b lin + |s| p) / |s| = sign(s) 2^-b lin + p: lane groups 0..2
    // add the three parts of the linear term, group 3 holds zero there.
    t[l] = fmaf(sg, lin[l], p);
  }
  asm volatile("" ::"v"(lin[3]));  // keeps the unread element's register from reuse (as in the f16 kernel)
  if constexpr (PER_LAYER) {
    (void)store_tile<MEAN, true>(cx, t, fabsf(s), tile);
  } else {
    x[(P + 7) & 3] = tile_rows<MEAN>(t, fabsf(s));
    if (P == 0 || P == 4) store_group(cx, group_scores<MEAN>(cx, x), tile - 3);
  }
}

// Instruction order of one phase: every MFMA followed by up to four
// vector-ALU instructions (the reduction of the previous tile, about 84 per
// tile, so none is left after the last MFMA), then the phase's requests and
// stores; nothing crosses a phase boundary.  Measured per tile in shader
// clocks: three per MFMA 1017 (the sigmoid chain then runs after the last
// MFMA), four 906, five 940, six 1000; requests placed earlier in the
// phase cost more.
__device__ __forceinline__ void interleave_phase8() {
#pragma unroll
  for (int k = 0; k < kLayers * 4 * 2 + 1; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);    // VMEM read: codes, scale
  __builtin_amdgcn_sched_group_barrier(0x040, 4, 0);    // VMEM write
  __builtin_amdgcn_sched_barrier(0);
}

// One pipeline run over chunks [start, start + count) of row b (every chunk
// below the row's valid_n).  In the phase of tile i the wave issues the 25
// MFMAs of tile i straight from its ring slot, the reduction of tile i-1,
// and the request of tile i+6 (6 tiles in flight).  Tiles past the run's
// chunks read as zeros and their stores are dropped.
template <bool MEAN, bool PER_LAYER>
__device__ __forceinline__ void score_run8(const i32x8* __restrict__ qpack8, const float* __restrict__ w8,
                                           const uint8_t* __restrict__ comp_k, int B, int64_t N, int b, int64_t start,
                                           int64_t count, int lane, float* __restrict__ scores,
                                           float* __restrict__ per_layer) {
  const Ctx cx = make_ctx<PER_LAYER>(comp_k, B, N, b, start, count, lane, scores, per_layer);

  i32x8 qh[kLayers][4], ql[kLayers][4];
  i32x8 qlin;
  f32x4 wv[kLayers][4];
  int32_t qsc;  // the linear fragment's A block-scale code (2^-b_l)
  {
    const i32x8* qp = qpack8 + (size_t)b * kQ8Frags * 64 + lane;
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        qh[l][mt] = qp[((l * 4 + mt) * 2) * 64];
        ql[l][mt] = qp[((l * 4 + mt) * 2 + 1) * 64];
      }
    qlin = qp[kQ8HeadFrags * 64];
    const float* wb = w8 + (size_t)b * kW8Row;
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) wv[l][mt] = *(const f32x4*)(wb + l * kHeads + 16 * mt + 4 * cx.g);
    qsc = ((const int32_t*)(wb + kLayers * kHeads))[lane];
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
  // Query parts in accumulation registers (the MFMA reads A from there);
  // the weights consumed before the loop, so their wait is paid here.
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      asm volatile("" : "+a"(qh[l][mt]));
      asm volatile("" : "+a"(ql[l][mt]));
    }
  asm volatile("" : "+a"(qlin));
#pragma unroll
  for (int l = 0; l < kLayers; ++l) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) asm volatile("" : "+v"(wv[l][mt]));
  }
  asm volatile("" : "+v"(qsc));

  const int tiles = (int)((count + kTile - 1) / kTile);

  f32x4 acc[2][kLayers][4];
  f32x4 lin[2];
  float x[4] = {0.f, 0.f, 0.f, 0.f};  // tile_rows of the open group's tiles

  // Phase of tile i, P = i mod 8: MFMAs of tile i from its ring slot; finish
  // tile i-1 (its scale still in its slot); request tile i+6 into the slot of
  // tile i-2, finished in the previous phase.
#define FM_PHASE8(P, I)                                                                                   \
  {                                                                                                       \
    mfma_tile8(qh, ql, qlin, qsc, tile_codes(ring[(P) & 7]), acc[(P) & 1], lin[(P) & 1]);                      \
    finish_tile8<MEAN, PER_LAYER, P>(cx, acc[((P) + 1) & 1], lin[((P) + 1) & 1], wv,                     \
                                     ring[((P) + 7) & 7].s, (I) - 1, x);                                  \
    load_tile(cx, (I) + kAhead, ring[((P) + 6) & 7]);                                                     \
    interleave_phase8();                                                                                  \
  }

  mfma_tile8(qh, ql, qlin, qsc, tile_codes(ring[0]), acc[0], lin[0]);
  load_tile(cx, kAhead, ring[kAhead]);

  // Tiles 1 .. 8 m, eight per iteration, branch-free (tiles past the last
  // valid one read zeros and their stores are dropped).
  int i = 1;
  do {
    FM_PHASE8(1, i)
    FM_PHASE8(2, i + 1)
    FM_PHASE8(3, i + 2)
    FM_PHASE8(4, i + 3)
    FM_PHASE8(5, i + 4)
    FM_PHASE8(6, i + 5)
    FM_PHASE8(7, i + 6)
    FM_PHASE8(0, i + 7)
    i += 8;
  } while (i < tiles);
  // Tile i - 1 (0 mod 8); with scores only, it opens a group whose other
  // tiles are past the run.
  finish_tile8<MEAN, PER_LAYER, 1>(cx, acc[0], lin[0], wv, ring[0].s, i - 1, x);
  if constexpr (!PER_LAYER) store_group(cx, group_scores<MEAN>(cx, x), i - 1);
#undef FM_PHASE8
}

// grid = number of compute units, block = 256 (one wave per SIMD); each wave
// scores its share of the tile list (walk_share).
template <bool MEAN, bool PER_LAYER>
__global__ __launch_bounds__(256, 1) void score8_kernel(const i32x8* __restrict__ qpack8, const float* __restrict__ w8,
                                                        const uint8_t* __restrict__ comp_k, int B, int64_t N,
                                                        const int32_t* __restrict__ valid_n,
                                                        const int64_t* __restrict__ row_tiles,
                                                        const int32_t* __restrict__ wave_row, int64_t total_tiles,
                                                        float* __restrict__ scores, float* __restrict__ per_layer) {
  const int lane = threadIdx.x & 63;
  walk_share(B, N, valid_n, row_tiles, wave_row, total_tiles, [&](int b, int64_t start, int64_t count) {
    score_run8<MEAN, PER_LAYER>(qpack8, w8, comp_k, B, N, b, start, count, lane, scores, per_layer);
  });
}

}  // namespace

hipError_t launch_score_fp8(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B,
                            int64_t N, const int32_t* valid_n, int mode, float* scores, float* per_layer,
                            hipStream_t stream) {
  hipLaunchKernelGGL(pack_q8_kernel, dim3(B * kLayers), dim3(256), 0, stream, q, w, B, (uint4*)ws.qpack8, ws.w8);
  const int64_t* row_tiles;
  int64_t total_tiles;
  hipError_t e = launch_score_plan(ws, valid_n, B, N, scores, per_layer, stream, &row_tiles, &total_tiles);
  if (e != hipSuccess) return e;
  const bool mean = mode == FM_ENSEMBLE_MEAN;
  auto kern = mean ? (per_layer ? score8_kernel<true, true> : score8_kernel<true, false>)
                   : (per_layer ? score8_kernel<false, true> : score8_kernel<false, false>);
  record_score_event(ws, 0, stream);
  hipLaunchKernelGGL(kern, dim3(ws.score_blocks), dim3(256), 0, stream, (const i32x8*)ws.qpack8, (const float*)ws.w8,
                     comp_k, B, N, valid_n, row_tiles, (const int32_t*)ws.wave_row, total_tiles, scores, per_layer);
  record_score_event(ws, 1, stream);
  return hipGetLastError();
}

}  // namespace fm
