// Query and weight branches of the Memory-Indexer (FlashMemory DS-V4
// Retriever README, "Architecture"):
//   a      = wq_a hidden                      (Q_LORA_RANK)
//   a_hat  = RMSNorm(a) * q_norm_weight       (eps inside the root)
//   q_lin  = wq_b a_hat, viewed [N_HEADS][HEAD_DIM] head-major
//   q      = Hadamard(RoPE_YaRN(q_lin))       (RoPE on the last 64 dims)
//   w      = weights_proj hidden * HEAD_DIM^-0.5 N_HEADS^-0.5
//
// The projections are skinny fp32 GEMMs (B <= a few dozen rows against up
// to 8192 weight rows), bound by streaming the weights from HBM.  Each fp32
// product x . w is formed on the f16 MFMA from two-part operands: at
// context creation every weight row is scaled by a power of two (its
// largest entry lands in [2^14, 2^15)) and split into f16 hi + lo parts (4
// bytes per weight, like fp32); each 128-wide chunk of an activation row is
// scaled and split the same way while it is staged.  Then
//   x w = xh wh + xh wl + xl wh  (+ xl wl, about 2^-22 relative, dropped)
// on three MFMAs, accumulated in fp32, and the scales are undone exactly.
// The fp32 MFMA would do the same work in about five times the cycles.
#include "fm_internal.h"

#include <cmath>

namespace fm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

// Power-of-two exponent e with m * 2^e in [2^14, 2^15) (0 for m == 0),
// clamped so that 2^e and 2^-e stay normal floats.
__device__ inline int split_exponent(float m) {
  if (!(m > 0.f)) return 0;
  int ex;
  (void)frexpf(m, &ex);  // m = f 2^ex, f in [0.5, 1)
  const int e = 15 - ex;
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}

// Packed weight layout, per layer: 16-row tiles; tile t holds K / 32
// k-steps of 2 KB each, k-step s = the MFMA A operands of rows 16 t .. 16 t
// + 15, k = 32 s .. 32 s + 31: 1 KB of hi parts then 1 KB of lo parts, lane
// l = i + 16 g (row 16 t + i, k = 32 s + 8 g .. + 7) at 16 l.  A wave's
// share of a tile is one contiguous stream.
__device__ inline size_t packed_offset(int row, int k, int K) {  // in halves, of the hi part of 8 k
  const int t = row >> 4, i = row & 15, s = k >> 5, g = (k >> 3) & 3;
  return ((size_t)(t * (K >> 5) + s) * 2) * 512 + (size_t)(i + 16 * g) * 8;
}

// One block per weight row: row * 2^e split into hi/lo f16 parts, written
// to the packed layout, and 2^-e.
__global__ __launch_bounds__(256) void pack_rows_kernel(const float* __restrict__ src, int K, int row0,
                                                        _Float16* __restrict__ packed, float* __restrict__ inv) {
  __shared__ float red[4];
  const float* row = src + (size_t)blockIdx.x * K;
  float m = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) m = fmaxf(m, fabsf(row[k]));
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = split_exponent(m);
  const float sc = ldexpf(1.f, e);
  const int r = row0 + blockIdx.x;
  for (int k8 = threadIdx.x * 8; k8 < K; k8 += 256 * 8) {
    f16x8 h, l;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float v = row[k8 + q] * sc;
      h[q] = (_Float16)v;
      l[q] = (_Float16)(v - (float)h[q]);
    }
    const size_t o = packed_offset(r, k8, K);
    *(f16x8*)(packed + o) = h;
    *(f16x8*)(packed + o + 512) = l;
  }
  if (threadIdx.x == 0) inv[r] = ldexpf(1.f, -e);
}

struct ProjArgs {
  const _Float16* w[kLayers];    // packed weights of each layer (layout above)
  const float* winv[kLayers];    // [rows]: 2^-e of each row
  const float* x;                // activations: x + layer * x_layer_stride + b * K
  float* out;                    // out[split][layer][b][rows]
  long x_layer_stride;
  int rows, K, B;  // K slices of kSliceK (grid y = layers * K / kSliceK)
};

// C[o][b] = sum_k W[o][k] x[b][k] on 16x16x32 f16 MFMA tiles (A = weights,
// rows = 16 outputs; B = activations, columns = 16 batch rows).  A block of
// 4 waves owns 64 consecutive outputs x 32 batch rows over one 512-wide K
// slice.  The slice's activations are staged once: all loads issued
// together, each 128-wide chunk of a row scaled by its own power of two and
// split into f16 hi/lo in LDS, one barrier.  Then each wave streams its own
// 16 weight rows through a ring of three register buffers (the weights of
// chunk c+2 requested before chunk c is multiplied), with no further
// barrier.
//
// MFMA operand layout (16x16x32 f16): lane l supplies A[l%16][8(l/16) + e]
// and B[8(l/16) + e][l%16], e = 0..7, and receives C[4(l/16) + r][l%16].
// K-step s covers k = 32 s .. 32 s + 31; lane l's eight k slots are
// 32 s + 8(l/16) + e, one 16-byte load of each part.
constexpr int kKChunk = 128;
constexpr int kKSteps = kKChunk / 32;                         // MFMA k-steps per chunk
constexpr int kXsStride = kSliceK + 8;                        // padded LDS row (halves)
constexpr int kStage = kProjRowsPerWave * kKChunk / 4 / 256;  // float4 activation loads per thread per chunk
constexpr int kWRing = 3;                                     // weight chunks in registers (two in flight)
constexpr int kProjLds = 2 * kProjRowsPerWave * kXsStride * 2 + kSliceChunks * kProjRowsPerWave * 4;

struct ProjLane {
  __amdgpu_buffer_rsrc_t w;  // this wave's 16-row tile (empty past the last row)
  __amdgpu_buffer_rsrc_t x;  // activation rows [0, B) of the layer
  int K, b_base;
};

struct WChunk {
  f16x8 hi[kKSteps], lo[kKSteps];
};

// K-step s of chunk kc is the 2 KB block kc / 32 + s of the wave's tile;
// the wave-uniform block offset goes in the scalar offset.
__device__ __forceinline__ void proj_load_w(const ProjLane& pl, int kc, WChunk& wc) {
  const uint32_t lane_off = 16u * (threadIdx.x & 63);
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) {
    const int so = 2048 * ((kc >> 5) + s);
    wc.hi[s] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(pl.w, lane_off, so, 0));
    wc.lo[s] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(pl.w, lane_off + 1024, so, 0));
  }
}

// Load j of wave v (of a group of four staging one slice) covers batch
// rows 8 j + 2 v (lanes 0..31) and 8 j + 2 v + 1 (lanes 32..63), one float4
// per lane.
__device__ __forceinline__ int stage_row(int j) {
  return 8 * j + 2 * (int)((threadIdx.x >> 6) & 3) + ((threadIdx.x >> 5) & 1);
}

// Activation rows b_base .. b_base + 32 (zeros past B) of the slice's
// chunk c, to registers.  The per-lane offset holds the row (so rows past B
// read zeros), the scalar offset the slice column.
__device__ __forceinline__ void proj_load_x(const ProjLane& pl, int k0, f32x4 (&xr)[kStage]) {
  const int c4 = threadIdx.x & 31;
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const uint32_t off = 4u * ((uint32_t)(pl.b_base + stage_row(j)) * pl.K + 4 * c4);
    xr[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pl.x, off, 4 * k0, 0));
  }
}

// Largest value over each group of 32 lanes (lanes 0..31 and 32..63), every
// lane of the group receiving it: DPP moves within rows of 16 lanes (quad
// swaps, then the half-row and row mirrors pair each lane with one of the
// other half), then a swap of neighbouring rows.  All in the vector ALU, no
// LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float max32(float m) {
  m = fmaxf(m, dpp_move<0xb1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp_move<0x4e>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp_move<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp_move<0x140>(m));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Chunk c of each staged row: scaled by its power of two (from its largest
// entry, a reduction over the 32 lanes holding it), split into f16 hi/lo,
// stored to LDS columns 128 c .. with the row's 2^-e.
__device__ __forceinline__ void proj_store_x(const f32x4 (&xr)[kStage], int c, _Float16* xs_hi, _Float16* xs_lo,
                                             float* xs_inv) {
  const int c4 = threadIdx.x & 31;
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const f32x4 v = xr[j];
    const float m = max32(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    const int e = split_exponent(m);
    const float sc = ldexpf(1.f, e);
    f16x4 h, l;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float y = v[q] * sc;
      h[q] = (_Float16)y;
      l[q] = (_Float16)(y - (float)h[q]);
    }
    const int row = stage_row(j);
    *(f16x4*)(xs_hi + row * kXsStride + kKChunk * c + 4 * c4) = h;
    *(f16x4*)(xs_lo + row * kXsStride + kKChunk * c + 4 * c4) = l;
    if (c4 == 0) xs_inv[c * kProjRowsPerWave + row] = ldexpf(1.f, -e);
  }
}

// Chunk c: three product terms on separate accumulators (six independent
// MFMA chains), then the chunk's sum times the batch row's 2^-e into tot.
template <int BT>
__device__ __forceinline__ void proj_chunk(const WChunk& wc, int c, const _Float16* xs_hi, const _Float16* xs_lo,
                                           const float* xs_inv, int i, int g, f32x4 (&tot)[BT]) {
  f32x4 hh[BT], hl[BT], lh[BT];
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) hh[bt] = hl[bt] = lh[bt] = zero;
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) {
    f16x8 xh[BT], xl[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) {
      const int o = (16 * bt + i) * kXsStride + kKChunk * c + 32 * s + 8 * g;
      xh[bt] = *(const f16x8*)(xs_hi + o);
      xl[bt] = *(const f16x8*)(xs_lo + o);
    }
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) hh[bt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wc.hi[s], xh[bt], hh[bt], 0, 0, 0);
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) hl[bt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wc.hi[s], xl[bt], hl[bt], 0, 0, 0);
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) lh[bt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wc.lo[s], xh[bt], lh[bt], 0, 0, 0);
  }
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) {
    const float sx = xs_inv[c * kProjRowsPerWave + 16 * bt + i];  // C column = batch row 16 bt + l%16
    tot[bt] += (hh[bt] + (hl[bt] + lh[bt])) * sx;
    // Fold the chunk in here: left alone, the compiler sinks every chunk's
    // update to the final store and keeps all the chunk sums alive.
    asm volatile("" : "+v"(tot[bt]));
  }
}

// Workgroup barrier ordering LDS only: weight loads already issued stay in
// flight across it (a full barrier would drain them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// grid = (outputs / (64 T), layers * K / 512, row groups), block = 256,
// dynamic LDS kProjLds.  Each wave takes T consecutive 16-row tiles over the
// block's K slice, one after the other: the weight ring runs on across the
// tiles, so a wave streams T x 4 chunks.  The first projection (408 blocks,
// within one round of two resident blocks per compute unit) uses T = 1.
template <int T>
__global__ __launch_bounds__(256, 2) void proj_kernel(ProjArgs p) {
  constexpr int BT = kProjRowsPerWave / 16;
  constexpr int kChunks = T * kSliceChunks;
  extern __shared__ __attribute__((aligned(16))) unsigned char proj_lds[];
  _Float16* xs_hi = (_Float16*)proj_lds;
  _Float16* xs_lo = xs_hi + kProjRowsPerWave * kXsStride;
  float* xs_inv = (float*)(xs_lo + kProjRowsPerWave * kXsStride);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int o_first = (blockIdx.x * 4 + wave) * 16 * T;
  const int splits = p.K / kSliceK;
  const int layer = blockIdx.y / splits;
  const int split = blockIdx.y % splits;
  const int k_begin = split * kSliceK;
  const int i = lane & 15;
  const int g = lane >> 4;

  ProjLane pl[T];
  {
    // Static indices and readfirstlane keep the descriptors in scalar
    // registers (a vector-register descriptor costs a loop per load).
    const _Float16* wl = layer == 0 ? p.w[0] : (layer == 1 ? p.w[1] : p.w[2]);
    const size_t tile_halves = (size_t)16 * p.K * 2;
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const int o_base = o_first + 16 * tt;
      const uint64_t a = (uint64_t)(uintptr_t)(wl + (size_t)(o_base >> 4) * tile_halves);  // never read past the rows
      const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
      const int bytes = __builtin_amdgcn_readfirstlane(o_base < p.rows ? (int)(tile_halves * 2) : 0);
      pl[tt].w = __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)u, 0, bytes, kBufferWord3);
      pl[tt].x = __builtin_amdgcn_make_buffer_rsrc((void*)(p.x + layer * p.x_layer_stride), 0, p.B * p.K * 4,
                                                   kBufferWord3);
      pl[tt].K = p.K;
      pl[tt].b_base = blockIdx.z * kProjRowsPerWave;
    }
  }

  // Chunk q of the wave's stream: tile q / 4, K chunk q % 4 of the slice.
  WChunk wbuf[kWRing];
#pragma unroll
  for (int q = 0; q < kWRing - 1; ++q)
    proj_load_w(pl[q / kSliceChunks], k_begin + (q % kSliceChunks) * kKChunk, wbuf[q]);
  {
    f32x4 xr[kSliceChunks][kStage];
#pragma unroll
    for (int c = 0; c < kSliceChunks; ++c) proj_load_x(pl[0], k_begin + c * kKChunk, xr[c]);
#pragma unroll
    for (int c = 0; c < kSliceChunks; ++c) proj_store_x(xr[c], c, xs_hi, xs_lo, xs_inv);
  }
  lds_barrier();

#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    f32x4 tot[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) tot[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kSliceChunks; ++c) {
      const int q = tt * kSliceChunks + c;
      if (q + kWRing - 1 < kChunks) {
        const int qn = q + kWRing - 1;
        proj_load_w(pl[qn / kSliceChunks], k_begin + (qn % kSliceChunks) * kKChunk, wbuf[qn % kWRing]);
      }
      proj_chunk<BT>(wbuf[q % kWRing], c, xs_hi, xs_lo, xs_inv, i, g, tot);
      __builtin_amdgcn_sched_barrier(0);  // keep each chunk's loads with it (registers)
    }

    // C rows are outputs, C columns batch rows: lane l holds o = o_base +
    // 4(l/16) + r, r = 0..3, for batch row 16 bt + l%16.  Undo the weight
    // rows' scales and store the four consecutive outputs.
    const int o = o_first + 16 * tt + 4 * g;
    if (o < p.rows) {
      const float* inv = layer == 0 ? p.winv[0] : (layer == 1 ? p.winv[1] : p.winv[2]);
      const f32x4 sw = *(const f32x4*)(inv + o);
#pragma unroll
      for (int bt = 0; bt < BT; ++bt) {
        const int b = pl[0].b_base + 16 * bt + i;
        if (b < p.B) *(f32x4*)(p.out + (((size_t)split * kLayers + layer) * p.B + b) * p.rows + o) = tot[bt] * sw;
      }
    }
  }
}

template <int T>
void launch_proj(const ProjArgs& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL(proj_kernel<T>, grid, dim3(256), kProjLds, stream, p);
}

// Sum over the 64 lanes, every lane receiving it: the max32 pattern with
// adds, then a swap of the wave's halves.
__device__ inline float wave_sum(float v) {
  v += dpp_move<0xb1>(v);
  v += dpp_move<0x4e>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct GainPtrs {
  const float* g[kLayers];
};

// cos and sin of phi = pos * freq.  phi reaches about 1e6 rad (positions up
// to 2^20, first frequency 1 rad/token), so it is formed and reduced to
// |r| <= pi in double precision: n = rint(phi / 2 pi), r = phi - n 2 pi with
// 2 pi split into a double (2PI_HI) and its remainder (2PI_LO), each product
// subtracted by one fused multiply-add (two-constant Cody-Waite reduction;
// n stays below 2^20, far inside the exact range).  The cosine and sine of
// the small r are then taken in single precision.
__device__ inline void rope_cos_sin(int64_t pos, double freq, float* out2) {
  const double two_pi_hi = 6.283185307179586;       // 2 pi rounded to double
  const double two_pi_lo = 2.4492935982947064e-16;  // 2 pi - two_pi_hi
  const double phi = (double)pos * freq;
  const double n = rint(phi * 0.15915494309189535);  // 1 / (2 pi)
  double r = fma(-n, two_pi_hi, phi);
  r = fma(-n, two_pi_lo, r);
  const float rf = (float)r;
  out2[0] = cosf(rf);
  out2[1] = sinf(rf);
}

// One 256-thread block per (layer, row): adds the K-slice partials in slice
// order, then RMSNorm (a / sqrt(mean(a^2) + eps) * gain) of the
// Q_LORA_RANK vector, and finishes the weight branch (weights_proj rows
// times weight_scale).  The layer-0 block of a row also stores the cosine
// and sine of the row's RoPE angles.
template <int S>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* part, GainPtrs gains, int B, float eps,
                                                      float w_scale, const int64_t* positions, const double* freq,
                                                      float* rope_cs, _Float16* ahat_hi, _Float16* ahat_lo,
                                                      float* ahat_inv, float* w_out) {
  const int layer = blockIdx.x / B;
  const int b = blockIdx.x % B;
  const int t = threadIdx.x;
  const size_t split_stride = (size_t)kLayers * B * kProj1Out;
  const float* src = part + ((size_t)layer * B + b) * kProj1Out;
  // Thread t owns outputs 4t .. 4t+3 (one float4 per slice); every slice's
  // load is issued before the first add.
  f32x4 sl[S];
#pragma unroll
  for (int s = 0; s < S; ++s) sl[s] = *(const f32x4*)(src + s * split_stride + 4 * t);
  float wpart[S];
  if (t < kHeads) {
#pragma unroll
    for (int s = 0; s < S; ++s) wpart[s] = src[s * split_stride + kQLora + t];
  }
  f32x4 a = sl[0];
#pragma unroll
  for (int s = 1; s < S; ++s) a += sl[s];
  float ss = a[0] * a[0];
  ss = fmaf(a[1], a[1], ss);
  ss = fmaf(a[2], a[2], ss);
  ss = fmaf(a[3], a[3], ss);
  ss = wave_sum(ss);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float rs = 1.0f / sqrtf(ss * (1.0f / kQLora) + eps);
  const float* gain = gains.g[layer];
  const f32x4 gv = {gain[4 * t], gain[4 * t + 1], gain[4 * t + 2], gain[4 * t + 3]};
  {
    // a_hat as wq_b's operand: each 128-chunk (32 lanes) scaled by the power
    // of two that puts its largest entry in [2^14, 2^15), split into f16
    // hi + lo, and the chunk's 2^-e.
    const f32x4 v = a * rs * gv;
    const float m = max32(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    const int e = split_exponent(m);
    const float sc = ldexpf(1.f, e);
    f16x4 h, l;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float y = v[q] * sc;
      h[q] = (_Float16)y;
      l[q] = (_Float16)(y - (float)h[q]);
    }
    const size_t o = ((size_t)layer * B + b) * kQLora + 4 * t;
    *(f16x4*)(ahat_hi + o) = h;
    *(f16x4*)(ahat_lo + o) = l;
    if ((t & 31) == 0) ahat_inv[((size_t)layer * B + b) * (kQLora / kKChunk) + (t >> 5)] = ldexpf(1.f, -e);
  }
  if (t < kHeads) {
    float wv = wpart[0];
#pragma unroll
    for (int s = 1; s < S; ++s) wv += wpart[s];
    w_out[((size_t)layer * B + b) * kHeads + t] = wv * w_scale;
  } else if (layer == 0 && t >= 64 && t < 64 + kRopeDim / 2) {
    const int j = t - 64;
    rope_cos_sin(positions[b], freq[j], rope_cs + ((size_t)b * (kRopeDim / 2) + j) * 2);
  }
}

// The value of lane l ^ M, for M = 1, 2, 4, 8, 16, 32: DPP lane moves in
// the vector ALU (quad permutes; row shifts by M from either side within
// each row of 16 lanes) and the gfx950 row swaps (permlane16/32_swap
// exchange the odd 16-lane rows of the first operand with the even rows of
// the second, or the wave's halves).
template <int M>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  if constexpr (M == 1) {
    return dpp_move<0xb1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return dpp_move<0x4e>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4 || M == 8) {
    const float up = dpp_move<0x100 + M>(v);    // row_shl:M, lane l receives lane l + M
    const float down = dpp_move<0x110 + M>(v);  // row_shr:M, lane l receives lane l - M
    return (lane & M) ? down : up;
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

template <int M>
__device__ __forceinline__ void butterfly(float& a0, float& a1, int lane) {
  const float p0 = xor_lane<M>(a0, lane);
  const float p1 = xor_lane<M>(a1, lane);
  const bool upper = lane & M;
  a0 = upper ? p0 - a0 : a0 + p0;
  a1 = upper ? p1 - a1 : a1 + p1;
}

// RoPE and the normalized Hadamard transform of one head's 128 dims, held
// by a wave as dims 2l and 2l+1 in lane l (x, y).  RoPE: lanes 32..63 hold
// the rotated dims 64..127; pair j = l - 32 is turned counter-clockwise by
// pos * freq[j] (cosine and sine from the RMSNorm kernel), the rotation in
// fp32.  Then the 128-point Walsh-Hadamard butterfly in Sylvester order
// (dims 2l, 2l+1 within the lane, then the lane bits), scaled by 128^-0.5.
__device__ __forceinline__ float2 rope_hadamard(float x, float y, const float* cs_row, int lane) {
  if (lane >= 32) {
    const float2 c = *(const float2*)(cs_row + 2 * (lane - 32));
    const float rx = x * c.x - y * c.y;
    const float ry = x * c.y + y * c.x;
    x = rx;
    y = ry;
  }
  float a0 = x + y;
  float a1 = x - y;
  butterfly<1>(a0, a1, lane);
  butterfly<2>(a0, a1, lane);
  butterfly<4>(a0, a1, lane);
  butterfly<8>(a0, a1, lane);
  butterfly<16>(a0, a1, lane);
  butterfly<32>(a0, a1, lane);
  const float inv_sqrt = 0.08838834764831845f;  // 128^-0.5
  return make_float2(a0 * inv_sqrt, a1 * inv_sqrt);
}

// q = Hadamard(RoPE(wq_b a_hat)) in one pass.  One block of 8 waves per
// (head, layer, group of 32 batch rows) computes the head's 128 outputs of
// wq_b over the whole K = Q_LORA_RANK: wave w takes K slice w / 4 and the
// 32 outputs 32 (w % 4) .. + 31 (two 16-row tiles, streamed one after the
// other through one register ring); both slices' activations are staged
// side by side in LDS.
// The two slices' sums meet in LDS (slice 0 + slice 1), and each wave then
// rotates, transforms and stores four batch rows.  The head's whole weight
// block (512 KB) is streamed by one compute unit, so no partial sums leave
// the block and no second launch is needed.
constexpr int kHeadThreads = 512;
constexpr int kHeadProjLds = 2 * kProjLds;
constexpr int kHeadRing = 3;  // weight chunks in registers per wave (kHeadRing - 1 in flight)
static_assert(kQLora == 2 * kSliceK, "two K slices per head block");
static_assert(2 * kProjRowsPerWave * kHeadDim * 4 <= kHeadProjLds, "slice sums fit in the staging area");

struct HeadProjArgs {
  const _Float16* w[kLayers];  // packed wq_b of each layer
  const float* winv[kLayers];  // [kHeads * kHeadDim]: 2^-e of each row
  const _Float16* ahat_hi;     // [3][B][kQLora], split a_hat (hi, lo parts)
  const _Float16* ahat_lo;
  const float* ahat_inv;       // [3][B][kQLora / 128]
  const float* rope_cs;        // [B][kRopeDim / 2][2]
  float* q_out;                // [3][B][kHeads][kHeadDim]
  int B;
};

__global__ __launch_bounds__(kHeadThreads, 1) void head_proj_kernel(HeadProjArgs p) {
  constexpr int BT = kProjRowsPerWave / 16;
  constexpr int T = 2;
  constexpr int kChunks = T * kSliceChunks;
  extern __shared__ __attribute__((aligned(16))) unsigned char head_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave >> 2;  // K slice
  const int head = blockIdx.x;
  const int layer = blockIdx.y;
  const int b_base = blockIdx.z * kProjRowsPerWave;
  _Float16* xs_hi = (_Float16*)(head_lds + half * kProjLds);
  _Float16* xs_lo = xs_hi + kProjRowsPerWave * kXsStride;
  float* xs_inv = (float*)(xs_lo + kProjRowsPerWave * kXsStride);
  const int k_begin = half * kSliceK;
  const int d_first = (wave & 3) * 16 * T;  // first of the wave's outputs within the head
  const int o_first = head * kHeadDim + d_first;
  const int i = lane & 15;
  const int g = lane >> 4;

  ProjLane pl[T];
  {
    const _Float16* wl = layer == 0 ? p.w[0] : (layer == 1 ? p.w[1] : p.w[2]);
    const size_t tile_halves = (size_t)16 * kQLora * 2;
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const uint64_t a = (uint64_t)(uintptr_t)(wl + (size_t)((o_first >> 4) + tt) * tile_halves);
      const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
      pl[tt].w = __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)u, 0, (int)(tile_halves * 2), kBufferWord3);
      pl[tt].K = kQLora;
      pl[tt].b_base = b_base;
    }
  }

  WChunk wbuf[kHeadRing];
#pragma unroll
  for (int q = 0; q < kHeadRing - 1; ++q)
    proj_load_w(pl[q / kSliceChunks], k_begin + (q % kSliceChunks) * kKChunk, wbuf[q]);
  {
    // The half's slice of the split a_hat rows b_base .. b_base + 31 (zeros
    // past B) copied to LDS: thread u of the half moves 16-byte vectors
    // u + 256 j of each part, vector v = row 64 ... column 8 (v % 64).
    const int u = threadIdx.x & 255;
    const size_t lo_row = (size_t)layer * p.B;
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.ahat_hi + lo_row * kQLora), 0, p.B * kQLora * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.ahat_lo + lo_row * kQLora), 0, p.B * kQLora * 2, kBufferWord3);
    constexpr int kVec = kProjRowsPerWave * kSliceK / 8 / 256;  // 16-byte vectors per thread and part
    f16x8 vh[kVec], vl[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v = u + 256 * j;
      const uint32_t off = 2u * ((uint32_t)(b_base + v / 64) * kQLora + k_begin + 8 * (v % 64));
      vh[j] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rh, off, 0, 0));
      vl[j] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rl, off, 0, 0));
    }
    float inv = 0.f;
    if (u < kSliceChunks * kProjRowsPerWave) {  // xs_inv[c][row], c = u / 32
      const int row = u % kProjRowsPerWave, c = u / kProjRowsPerWave;
      const int b = b_base + row;
      inv = b < p.B ? p.ahat_inv[(lo_row + b) * (kQLora / kKChunk) + k_begin / kKChunk + c] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v = u + 256 * j;
      *(f16x8*)(xs_hi + (v / 64) * kXsStride + 8 * (v % 64)) = vh[j];
      *(f16x8*)(xs_lo + (v / 64) * kXsStride + 8 * (v % 64)) = vl[j];
    }
    if (u < kSliceChunks * kProjRowsPerWave) xs_inv[u] = inv;
  }
  lds_barrier();

  f32x4 res[T][BT];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    f32x4 tot[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) tot[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kSliceChunks; ++c) {
      const int q = tt * kSliceChunks + c;
      if (q + kHeadRing - 1 < kChunks) {
        const int qn = q + kHeadRing - 1;
        proj_load_w(pl[qn / kSliceChunks], k_begin + (qn % kSliceChunks) * kKChunk, wbuf[qn % kHeadRing]);
      }
      proj_chunk<BT>(wbuf[q % kHeadRing], c, xs_hi, xs_lo, xs_inv, i, g, tot);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Lane l holds outputs o = o_first + 16 tt + 4(l/16) + r for batch row
    // 16 bt + l%16; undo the weight rows' scales.
    const float* inv = layer == 0 ? p.winv[0] : (layer == 1 ? p.winv[1] : p.winv[2]);
    const f32x4 sw = *(const f32x4*)(inv + o_first + 16 * tt + 4 * g);
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) res[tt][bt] = tot[bt] * sw;
  }

  // Slice sums to LDS (over the staging area, once every wave is done with
  // it): sums[half][batch row][dim].
  lds_barrier();
  float* sums = (float*)head_lds;
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
      *(f32x4*)(sums + ((size_t)half * kProjRowsPerWave + 16 * bt + i) * kHeadDim + d_first + 16 * tt + 4 * g) =
          res[tt][bt];
  lds_barrier();

  // Wave w finishes batch rows w, w + 8, w + 16, w + 24 of the group.
#pragma unroll
  for (int j = 0; j < kProjRowsPerWave / 8; ++j) {
    const int r = wave + 8 * j;
    const int b = b_base + r;
    if (b >= p.B) break;
    const float2 s0 = *(const float2*)(sums + (size_t)r * kHeadDim + 2 * lane);
    const float2 s1 = *(const float2*)(sums + ((size_t)kProjRowsPerWave + r) * kHeadDim + 2 * lane);
    const float2 v = rope_hadamard(s0.x + s1.x, s0.y + s1.y, p.rope_cs + (size_t)b * kRopeDim, lane);
    *(float2*)(p.q_out + (((size_t)layer * p.B + b) * kHeads + head) * kHeadDim + 2 * lane) = v;
  }
}

}  // namespace

hipError_t launch_prepare_query(const fm_config& cfg, const fm_weights& wts, const Workspace& ws, int max_batch,
                                const float* hidden, const int64_t* positions, int B, float* q_out, float* w_out,
                                hipStream_t stream) {
  (void)max_batch;
  (void)wts;  // packed into the workspace by fm_create
  const int row_groups = proj_row_groups(B);
  const int s1 = kHidden / kSliceK;

  // wq_a | weights_proj (packed together), split over K.
  {
    ProjArgs p{};
    for (int l = 0; l < kLayers; ++l) {
      p.w[l] = ws.w1 + (size_t)l * kProj1Out * kHidden * 2;
      p.winv[l] = ws.w1_inv + (size_t)l * kProj1Out;
    }
    p.x = hidden;
    p.x_layer_stride = 0;
    p.out = ws.proj1_part;
    p.rows = kProj1Out;
    p.K = kHidden;
    p.B = B;
    const int col_tiles = (kProj1Out + 15) / 16;
    dim3 grid((col_tiles + 3) / 4, kLayers * s1, row_groups);
    launch_proj<1>(p, grid, stream);
  }
  // RMSNorm + weight-branch finish + RoPE angles.
  {
    GainPtrs gp{};
    for (int l = 0; l < kLayers; ++l) gp.g[l] = ws.q_norm + (size_t)l * kQLora;
    const float w_scale = (float)(1.0 / std::sqrt((double)cfg.head_dim * (double)cfg.n_heads));
    auto kern = rmsnorm_kernel<kHidden / kSliceK>;
    hipLaunchKernelGGL(kern, dim3(kLayers * B), dim3(256), 0, stream, ws.proj1_part, gp, B, cfg.rms_eps, w_scale,
                       positions, ws.rope_freq, ws.rope_cs, ws.ahat_hi, ws.ahat_lo, ws.ahat_inv, w_out);
  }
  // wq_b, RoPE (YaRN) and the normalized Hadamard transform, per head.
  {
    HeadProjArgs p{};
    for (int l = 0; l < kLayers; ++l) {
      p.w[l] = ws.w2 + (size_t)l * kHeads * kHeadDim * kQLora * 2;
      p.winv[l] = ws.w2_inv + (size_t)l * kHeads * kHeadDim;
    }
    p.ahat_hi = ws.ahat_hi;
    p.ahat_lo = ws.ahat_lo;
    p.ahat_inv = ws.ahat_inv;
    p.rope_cs = ws.rope_cs;
    p.q_out = q_out;
    p.B = B;
    hipLaunchKernelGGL(head_proj_kernel, dim3(kHeads, kLayers, row_groups), dim3(kHeadThreads), kHeadProjLds, stream,
                       p);
  }
  return hipGetLastError();
}

hipError_t launch_pack_weights(const fm_weights& wts, const Workspace& ws, hipStream_t stream) {
  // The projection kernel stages a 512-wide slice of 32 activation rows
  // (about 66 KB of LDS, above the default dynamic limit).
  hipError_t a = hipFuncSetAttribute((const void*)proj_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, kProjLds);
  if (a == hipSuccess)
    a = hipFuncSetAttribute((const void*)head_proj_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kHeadProjLds);
  if (a != hipSuccess) return a;
  for (int l = 0; l < kLayers; ++l) {
    _Float16* w1 = ws.w1 + (size_t)l * kProj1Out * kHidden * 2;
    float* i1 = ws.w1_inv + (size_t)l * kProj1Out;
    hipLaunchKernelGGL(pack_rows_kernel, dim3(kQLora), dim3(256), 0, stream, wts.wq_a[l], kHidden, 0, w1, i1);
    hipLaunchKernelGGL(pack_rows_kernel, dim3(kHeads), dim3(256), 0, stream, wts.w_proj[l], kHidden, kQLora, w1, i1);
    hipLaunchKernelGGL(pack_rows_kernel, dim3(kHeads * kHeadDim), dim3(256), 0, stream, wts.wq_b[l], kQLora, 0,
                       ws.w2 + (size_t)l * kHeads * kHeadDim * kQLora * 2, ws.w2_inv + (size_t)l * kHeads * kHeadDim);
    hipError_t e = hipMemcpyAsync(ws.q_norm + (size_t)l * kQLora, wts.q_norm[l], sizeof(float) * kQLora,
                                  hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace fm
