// Per-layer chunk score and ensemble (FlashMemory DS-V4 Retriever README,
// "compressed_k format", "Architecture" score line, "Joint checkpoint +
// ensemble"):
//   k       = e4m3(bytes[0:128]) * f32le(bytes[128:132])
//   S_l     = sigmoid( sum_h relu(k . q_{l,h}) * w_{l,h} ),  l = l10, l12, l20
//   E       = max_l S_l  or  mean_l S_l
//
// Per request row this is a [N x 128] x [128 x 192] contraction (3 layers x
// 64 heads), 49152 flop per 132-byte chunk, on the 16x16x32 f16 MFMA
// (plus one 16x16x128 fp8 MFMA per 16 chunks for the linear term below).
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
//     one more MFMA per tile, on the fp8 matrix core with the stored e4m3
//     codes as they are (no decode) and the weighted query sum of each layer
//     scaled by a power of two and split into three e4m3 parts (about 15
//     bits below the largest element).  The second is one fused multiply-add
//     per head with an absolute-value operand, and a scale of either sign
//     costs nothing;
//   - max ensemble: max_l sigmoid(t_l) = sigmoid(max_l t_l), one sigmoid.
#include <algorithm>

#include "fm_score_common.h"

namespace fm {
namespace {

using namespace score;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// MFMA 16x16x32 f16 operand layout: lane l supplies A[l%16][8(l/16) + e] and
// B[8(l/16) + e][l%16], e = 0..7, and receives C[4(l/16) + r][l%16].
// A = queries (rows = 16 heads of a head tile), B = keys (columns = 16
// chunks).  For k-step t (t = 0..3) lane l's eight k slots are the dims
// 32(l/16) + 8t + e, so each lane reads one contiguous 32-byte run of its
// chunk's codes.  Fragment f = (layer * 4 + head_tile) * 4 + t for the
// heads.
//
// The linear term uses the 16x16x128 fp8 MFMA, whose lane l supplies
// A[l%16][32(l/16) + e] and B[32(l/16) + e][l%16], e = 0..31: B is lane
// l's 32 stored code bytes as they are.  Row 4k + l (k = 0..2, l = layer)
// of its A holds part k of u_l = 2^b_l v_l, v_l = 1/2 sum_h w_{l,h} q_{l,h}
// (q already rounded to f16, the sum in fp32), with 2^b_l putting the
// largest |u_l| in [128, 256): part 0 = e4m3(u), part 1 = e4m3(u - part 0),
// part 2 = e4m3 of what remains.  Other rows are zero.  The A operand's
// block scales (E8M0, one per row and 32-wide block, from the lane holding
// the block; code 127 is 1, checked on the GPU) undo 2^b_l: the rows of
// layer l carry code 127 - b_l.  The MFMA output then holds, in lane group
// k, part k of layer r's term in element r, already times 2^-b_l, and the
// cross-group sum adds the parts.
//
// Packed row: 48 head fragments (64 lanes x 16 bytes), the linear fragment
// (64 lanes x 32 bytes) at byte kQLinOffset, and each lane's A block-scale
// code (one int32 per lane) at byte kQScaleOffset.
constexpr int kQLinOffset = kQHeadFrags * 64 * 16;
constexpr int kQScaleOffset = kQLinOffset + 64 * 32;
static_assert(kQScaleOffset + 64 * 4 <= kQFrags * 64 * 16, "packed query row too small");

// 2^a with m 2^a in [128, 256) (m > 0); 0 for m = 0.
__device__ __forceinline__ int part_exponent(float m) {
  if (!(m > 0.f)) return 0;
  int ex;
  (void)frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
  return 8 - ex;
}

// One block per (row, layer), 256 threads.  Thread t packs the head
// fragments o = t + 256 j (j = 0..3; fragment o / 64, lane o % 64) from two
// float4 loads each, all issued first, and keeps the f16 queries in LDS;
// then v_d = 1/2 sum_h w_h q_hd is summed in two head halves (fp32), scaled
// by this layer's 2^b and split into three e4m3 parts scattered to this
// layer's rows of the linear fragment.  The layer-0 block also writes the
// zero rows.
__global__ __launch_bounds__(256) void pack_q_kernel(const float* __restrict__ q, const float* __restrict__ w, int B,
                                                     f16x8* __restrict__ qpack) {
  __shared__ __attribute__((aligned(16))) _Float16 qs[kHeads][kHeadDim + 8];
  __shared__ float red[2][kHeadDim];
  __shared__ float vmax[2];
  __shared__ __attribute__((aligned(16))) uint32_t lin8[3][kHeadDim / 4];  // [part][dims / 4]
  __shared__ float w_s[kHeads];  // the row's head weights, loaded with q (not in the sum's loop)
  const int b = blockIdx.x / kLayers;
  const int layer = blockIdx.x % kLayers;
  const int t = threadIdx.x;
  const float* qb = q + ((size_t)layer * B + b) * kHeads * kHeadDim;
  f16x8* out = qpack + (size_t)b * kQFrags * 64;
  const float wt = t < kHeads ? w[((size_t)layer * B + b) * kHeads + t] : 0.f;
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
  if (t < kHeads) w_s[t] = wt;
  __syncthreads();
  {
    const int d = t & (kHeadDim - 1), half = t >> 7;
    float acc = 0.f;
#pragma unroll 8
    for (int h = 0; h < 32; ++h) acc = fmaf(w_s[32 * half + h], (float)qs[32 * half + h][d], acc);
    red[half][d] = acc;
  }
  __syncthreads();
  float u = 0.f;
  if (t < kHeadDim) {
    u = 0.5f * (red[0][t] + red[1][t]);
    float mu = fabsf(u);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mu = fmaxf(mu, __shfl_xor(mu, off));
    if ((t & 63) == 0) vmax[t >> 6] = mu;
  }
  __syncthreads();
  uint8_t* row = (uint8_t*)out;
  if (t < kHeadDim) {
    const int bl = part_exponent(fmaxf(vmax[0], vmax[1]));
    float r = ldexpf(u, bl);
    uint32_t p[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      p[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.f, 0, false) & 0xffu;
      r -= __builtin_amdgcn_cvt_f32_fp8((int)p[k], 0);  // exact: p[k] is r rounded to 4 significant bits
    }
    // Gather the bytes of four consecutive dims into one word (lanes t..t+3).
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      uint32_t word = p[k] << (8 * (t & 3));
      word |= __shfl_xor(word, 1);
      word |= __shfl_xor(word, 2);
      if ((t & 3) == 0) lin8[k][t >> 2] = word;
    }
    // Block-scale codes of this layer's rows (rows 4k + layer, k = 0..2, in
    // all four lane groups); the layer-0 block also writes code 127 (scale
    // 1) for the zero rows.  2^-b_l below 2^-127 (|u_l| below 2^-119) is
    // clamped to 2^-127.
    const int r16 = t & 15;
    const bool mine = r16 < 12 && (r16 & 3) == layer;
    const bool zero_row = r16 >= 12 || (r16 & 3) == 3;
    const int code = 127 - bl < 0 ? 0 : (127 - bl > 254 ? 254 : 127 - bl);
    if (t < 64 && (mine || (layer == 0 && zero_row))) ((int32_t*)(row + kQScaleOffset))[t] = mine ? code : 127;
  }
  __syncthreads();
  uint4* lin_out = (uint4*)(row + kQLinOffset);
  if (t < 12) {  // part k = t / 4 of this layer, dims 32 j .. + 31 with j = t % 4
    const int k = t >> 2, j = t & 3;
    const int lane = 4 * k + layer + 16 * j;
    const uint4* src = (const uint4*)&lin8[k][8 * j];
    lin_out[2 * lane] = src[0];
    lin_out[2 * lane + 1] = src[1];
  }
  if (layer == 0 && t >= 16 && t < 16 + 28) {  // rows 3, 7, 11 .. 15 of every lane group
    const int z = (t - 16) >> 2, j = (t - 16) & 3;
    const int rw = z < 3 ? 4 * z + 3 : 9 + z;
    const int lane = rw + 16 * j;
    lin_out[2 * lane] = make_uint4(0, 0, 0, 0);
    lin_out[2 * lane + 1] = make_uint4(0, 0, 0, 0);
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

__device__ __forceinline__ i32x8 tile_codes(const RawTile& t) {
  return i32x8{(int)t.lo[0], (int)t.lo[1], (int)t.lo[2], (int)t.lo[3],
               (int)t.hi[0], (int)t.hi[1], (int)t.hi[2], (int)t.hi[3]};
}

// The 49 MFMAs of one tile: the linear term first (fp8, from the stored
// codes), then the 48 head MFMAs in k-step order, so no MFMA waits on the
// one before it.
__device__ __forceinline__ void mfma_tile(const f16x8 (&qf)[kLayers][4][4], const i32x8& qlin, int32_t qsc,
                                          const RawTile& raw, const f16x8 (&kf)[4], f32x4 (&acc)[kLayers][4],
                                          f32x4& lin) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // Format code 0 (e4m3) for both operands; A block scales qsc (2^-b_l),
  // B unscaled (code 127).
  lin = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qlin, tile_codes(raw), zero, 0, 0, 0, qsc, 0, 127);
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[l][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[l][mt][0], kf[0], zero, 0, 0, 0);
#pragma unroll
  for (int t = 1; t < 4; ++t) {
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[l][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[l][mt][t], kf[t], acc[l][mt], 0, 0, 0);
  }
}

// Head reduction, sigmoid, ensemble and store of one tile, in the phase
// P = (tile + 1) mod 8.  wh = w / 2; lin is already times 2^-b_l.
//
// Scores only (no per-layer output): tile_rows of the tile goes to
// x[tile mod 4], and the phase that finishes the last tile of an aligned
// group of four (P = 4 and 0) reduces, stores and, with the threshold mask
// folded in (THR), keeps the group's scores in e_pend; the next phase writes
// their mask (so it does not wait on this phase's chain).
//
// With per-layer scores: every tile is stored on its own, and with THR the
// mask of the tile before (its scores in e_pend) is written first.
template <bool MEAN, bool PER_LAYER, bool THR, int P>
__device__ __forceinline__ void finish_tile(const Ctx& cx, const f32x4 (&acc)[kLayers][4], const f32x4& lin,
                                            const f32x4 (&wh)[kLayers][4], float s, int tile, float& e_pend,
                                            float (&x)[4]) {
  if (THR && PER_LAYER) threshold_tile(cx, e_pend, tile - 1);
  if (THR && !PER_LAYER && (P == 1 || P == 5)) threshold_group(cx, e_pend, tile - 4);
  float t[kLayers];
  const float sg = __builtin_copysignf(1.0f, s);
#pragma unroll
  for (int l = 0; l < kLayers; ++l) {
    float p = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) p = fmaf(fabsf(acc[l][mt][r]), wh[l][mt][r], p);
    // (s 2^-b lin + |s| p) / |s| = sign(s) 2^-b lin + p: lane groups 0..2
    // add the three parts of the linear term, group 3 holds zero there.
    t[l] = fmaf(sg, lin[l], p);
  }
  // The linear term's fourth element is never read; keeping it live until
  // here stops its register being reused right after the MFMA that writes
  // it (a write-after-write wait on the 32-cycle MFMA).
  asm volatile("" ::"v"(lin[3]));
  if constexpr (PER_LAYER) {
    const float e = store_tile<MEAN, true>(cx, t, fabsf(s), tile);
    if (THR) e_pend = e;
  } else {
    x[(P + 7) & 3] = tile_rows<MEAN>(t, fabsf(s));
    if (P == 0 || P == 4) {
      const float e = group_scores<MEAN>(cx, x);
      store_group(cx, e, tile - 3);
      if (THR) e_pend = e;
    }
  }
}

// Instruction order of one phase for the scheduler: the fp8 MFMA (32
// cycles) followed by four vector-ALU instructions, every f16 MFMA (16
// cycles) by two (a wave issues in order, so the vector work of the
// reduction and decode must sit between the MFMAs to overlap them), then
// the phase's requests (after the decode has consumed the ring slot they
// refill) and its stores.
__device__ __forceinline__ void interleave_phase() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA (fp8 linear term)
  __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);    // VALU
#pragma unroll
  for (int k = 0; k < kLayers * 4 * 4; ++k) {
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
// issues the 49 MFMAs of tile i, interleaved with the reduction of tile i-1
// and the decode of tile i+1; the records of tile i+6 are requested in the
// same phase (6 tiles in flight).  Tiles past the run's chunks read as zeros
// and their stores are dropped by the buffer range checks.
template <bool MEAN, bool PER_LAYER, bool THR>
__device__ __forceinline__ void score_run(const f16x8* __restrict__ qpack, const float* __restrict__ w,
                                          const uint8_t* __restrict__ comp_k, int B, int64_t N, int b, int64_t start,
                                          int64_t count, int lane, float* __restrict__ scores,
                                          float* __restrict__ per_layer, uint8_t* __restrict__ mask, float threshold) {
  Ctx cx = make_ctx<PER_LAYER>(comp_k, B, N, b, start, count, lane, scores, per_layer);
  if (THR) {
    cx.mask = mask + (size_t)b * N + start;
    cx.threshold = threshold;
  }

  // Query fragments, the linear-term fragment and its scales, and w: every load is issued
  // before the first use, so the wave pays one memory latency here, not one
  // per fragment.
  f16x8 qf[kLayers][4][4];
  i32x8 qlin;
  f32x4 wv[kLayers][4];  // w / 2 of the heads this lane's accumulators hold: 16 mt + 4 g + r
  int32_t qsc;           // the linear fragment's A block-scale code (2^-b_l)
  {
    const f16x8* qrow = qpack + (size_t)b * kQFrags * 64;
    const f16x8* qp = qrow + lane;
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) qf[l][mt][t] = qp[((l * 4 + mt) * 4 + t) * 64];
    qlin = *((const i32x8*)((const uint8_t*)qrow + kQLinOffset) + lane);
    qsc = ((const int32_t*)((const uint8_t*)qrow + kQScaleOffset))[lane];
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
  asm volatile("" : "+a"(qlin));
  // Consume w here, so its wait is paid before the loop; a wait inside the
  // loop would also drain the records in flight.
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      wv[l][mt] = 0.5f * wv[l][mt];
      asm volatile("" : "+v"(wv[l][mt]));
    }
  asm volatile("" : "+v"(qsc));

  const int tiles = (int)((count + kTile - 1) / kTile);

  f16x8 kf[2][4];
  f32x4 acc[2][kLayers][4];
  f32x4 lin[2];
  float e_pend = 0.f;  // scores of the tile or group whose threshold mask is still to be written
  float x[4] = {0.f, 0.f, 0.f, 0.f};  // tile_rows of the open group's tiles

  // Phase of tile i, P = i mod 8 (compile-time, so every register index is
  // static): MFMAs of tile i; finish tile i-1 (its scale still in its ring
  // slot); decode tile i+1 (requested five phases ago); request tile i+6
  // into the slot of tile i-2, finished in the previous phase.
#define FM_PHASE(P, I)                                                                                \
  {                                                                                                   \
    mfma_tile(qf, qlin, qsc, ring[(P) & 7], kf[(P) & 1], acc[(P) & 1], lin[(P) & 1]);                \
    finish_tile<MEAN, PER_LAYER, THR, P>(cx, acc[((P) + 1) & 1], lin[((P) + 1) & 1], wv,              \
                                         ring[((P) + 7) & 7].s, (I) - 1, e_pend, x);                  \
    decode_tile(ring[((P) + 1) & 7], kf[((P) + 1) & 1]);                                              \
    load_tile(cx, (I) + kAhead, ring[((P) + 6) & 7]);                                                 \
    interleave_phase();                                                                               \
  }

  // Tile 0 (nothing to finish yet).
  decode_tile(ring[0], kf[0]);
  mfma_tile(qf, qlin, qsc, ring[0], kf[0], acc[0], lin[0]);
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
  // Tile i - 1 (0 mod 8); with scores only, it opens a group whose other
  // tiles are past the run (their stale rows in x go to dropped slots).
  finish_tile<MEAN, PER_LAYER, THR, 1>(cx, acc[0], lin[0], wv, ring[0].s, i - 1, e_pend, x);
  if constexpr (PER_LAYER) {
    if (THR) threshold_tile(cx, e_pend, i - 1);
  } else {
    const float e = group_scores<MEAN>(cx, x);
    store_group(cx, e, i - 1);
    if (THR) threshold_group(cx, e, i - 1);
  }
#undef FM_PHASE
}

// grid = number of compute units, block = 256 (one wave per SIMD); each wave
// scores its share of the tile list (walk_share).  THR: the threshold mask
// is written by the pass.
template <bool MEAN, bool PER_LAYER, bool THR>
__global__ __launch_bounds__(256, 1) void score_kernel(const f16x8* __restrict__ qpack, const float* __restrict__ w,
                                                       const uint8_t* __restrict__ comp_k, int B, int64_t N,
                                                       const int32_t* __restrict__ valid_n,
                                                       const int64_t* __restrict__ row_tiles,
                                                       const int32_t* __restrict__ wave_row,
                                                       int64_t total_tiles,  // used when row_tiles is null
                                                       float* __restrict__ scores, float* __restrict__ per_layer,
                                                       uint8_t* __restrict__ mask, float threshold) {
  const int lane = threadIdx.x & 63;
  walk_share(B, N, valid_n, row_tiles, wave_row, total_tiles, [&](int b, int64_t start, int64_t count) {
    score_run<MEAN, PER_LAYER, THR>(qpack, w, comp_k, B, N, b, start, count, lane, scores, per_layer, mask,
                                    threshold);
  });
}

// Plan for ragged rows (one block of 1024 threads): row_tiles[b] = sum of
// ceil(valid_n / 16) over the rows before b (row_tiles[B] = all tiles), and
// for each wave the row holding its first tile.
__device__ __forceinline__ void plan_rows(const int32_t* __restrict__ valid_n, int B, int64_t N, int waves,
                                          int64_t* __restrict__ row_tiles, int32_t* __restrict__ wave_row) {
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
    int64_t first, end;
    idx::wave_share(g, waves, total, &first, &end);
    wave_row[g] = idx::plan_row_of(s_pre, B, first);
  }
}

// Ragged rows, one launch before the score kernel (block = 1024 threads,
// grid = (tail_blocks + 1, B)): the last column's block of row 0 runs the
// plan (the other rows' blocks of that column have nothing to do); the
// other blocks write -inf for the chunks of row blockIdx.y at or beyond its
// valid_n (and, with the selection folded in, a zero mask byte).
template <bool PER_LAYER>
__global__ __launch_bounds__(1024) void score_ragged_kernel(const int32_t* __restrict__ valid_n, int B, int64_t N,
                                                            int waves, int64_t* __restrict__ row_tiles,
                                                            int32_t* __restrict__ wave_row, float* __restrict__ scores,
                                                            float* __restrict__ per_layer, uint8_t* __restrict__ mask) {
  const int tail_blocks = (int)gridDim.x - 1;
  if ((int)blockIdx.x == tail_blocks) {
    if (blockIdx.y == 0) plan_rows(valid_n, B, N, waves, row_tiles, wave_row);
    return;
  }
  const int b = blockIdx.y;
  const int64_t v = valid_n[b];
  const int64_t vn = v < 0 ? 0 : (v > N ? N : v);
  const float ninf = -__builtin_huge_valf();
  for (int64_t n = vn + (int64_t)blockIdx.x * 1024 + threadIdx.x; n < N; n += (int64_t)tail_blocks * 1024) {
    scores[(size_t)b * N + n] = ninf;
    if (PER_LAYER)
      for (int l = 0; l < kLayers; ++l) per_layer[((size_t)l * B + b) * N + n] = ninf;
    if (mask) mask[(size_t)b * N + n] = 0;
  }
}

// Threshold mask of each row's last N % 4 chunks: the score pass writes the
// mask in whole words and stops at the row's last whole word (runs start on
// 16-chunk tiles, so that word ends at N - N % 4 in every run of the row).
// grid = B, block = 64.
__global__ __launch_bounds__(64) void threshold_edge_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ valid_n, int64_t N,
                                                            float threshold, uint8_t* __restrict__ mask) {
  const int b = blockIdx.x;
  const int64_t n = (N & ~(int64_t)3) + threadIdx.x;
  if (n >= N) return;
  int64_t vn = N;
  if (valid_n) {
    const int64_t v = valid_n[b];
    vn = v < 0 ? 0 : (v > N ? N : v);
  }
  mask[(size_t)b * N + n] = (n < vn && scores[(size_t)b * N + n] > threshold) ? 1 : 0;
}

}  // namespace

namespace {

hipError_t plan_and_tail(const Workspace& ws, const int32_t* valid_n, int B, int64_t N, float* scores,
                         float* per_layer, uint8_t* mask, hipStream_t stream, const int64_t** row_tiles,
                         int64_t* total_tiles) {
  *total_tiles = (int64_t)B * ((N + kTile - 1) / kTile);
  *row_tiles = nullptr;
  if (valid_n) {
    *row_tiles = ws.row_tiles;
    const unsigned gx = (unsigned)std::min<int64_t>((N + 1023) / 1024, 16);  // tail blocks per row
    auto kern = per_layer ? score_ragged_kernel<true> : score_ragged_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(gx + 1, B), dim3(1024), 0, stream, valid_n, B, N, 4 * ws.score_blocks,
                       ws.row_tiles, ws.wave_row, scores, per_layer, mask);
  }
  return hipGetLastError();
}

template <bool THR>
hipError_t launch_score_sel(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B,
                            int64_t N, const int32_t* valid_n, int mode, float threshold, float* scores,
                            uint8_t* mask, float* per_layer, hipStream_t stream) {
  f16x8* qpack = (f16x8*)ws.qpack;
  hipLaunchKernelGGL(pack_q_kernel, dim3(B * kLayers), dim3(256), 0, stream, q, w, B, qpack);
  const int64_t* row_tiles;
  int64_t total_tiles;
  hipError_t e = plan_and_tail(ws, valid_n, B, N, scores, per_layer, THR ? mask : nullptr, stream, &row_tiles,
                               &total_tiles);
  if (e != hipSuccess) return e;
  const bool mean = mode == FM_ENSEMBLE_MEAN;
  auto kern = mean ? (per_layer ? score_kernel<true, true, THR> : score_kernel<true, false, THR>)
                   : (per_layer ? score_kernel<false, true, THR> : score_kernel<false, false, THR>);
  record_score_event(ws, 0, stream);
  hipLaunchKernelGGL(kern, dim3(ws.score_blocks), dim3(256), 0, stream, (const f16x8*)qpack, w, comp_k, B, N,
                     valid_n, row_tiles, (const int32_t*)ws.wave_row, total_tiles, scores, per_layer, mask,
                     threshold);
  record_score_event(ws, 1, stream);
  if (THR && (N & 3))
    hipLaunchKernelGGL(threshold_edge_kernel, dim3(B), dim3(64), 0, stream, (const float*)scores, valid_n, N,
                       threshold, mask);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_plan(const Workspace& ws, const int32_t* valid_n, int B, int64_t N, float* scores,
                             float* per_layer, hipStream_t stream, const int64_t** row_tiles, int64_t* total_tiles) {
  return plan_and_tail(ws, valid_n, B, N, scores, per_layer, nullptr, stream, row_tiles, total_tiles);
}

hipError_t launch_score(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B, int64_t N,
                        const int32_t* valid_n, int mode, float* scores, float* per_layer, hipStream_t stream) {
  return launch_score_sel<false>(ws, q, w, comp_k, B, N, valid_n, mode, 0.f, scores, nullptr, per_layer, stream);
}

hipError_t launch_score_threshold(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B,
                                  int64_t N, const int32_t* valid_n, int mode, float threshold, float* scores,
                                  uint8_t* mask, float* per_layer, hipStream_t stream) {
  return launch_score_sel<true>(ws, q, w, comp_k, B, N, valid_n, mode, threshold, scores, mask, per_layer, stream);
}

}  // namespace fm
