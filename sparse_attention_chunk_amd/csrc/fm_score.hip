// Per-layer chunk score and ensemble (FlashMemory DS-V4 Retriever README,
// "compressed_k format", "Architecture" score line, "Joint checkpoint +
// ensemble"):
//   k       = e4m3(bytes[0:128]) * f32le(bytes[128:132])
//   S_l     = sigmoid( sum_h relu(k . q_{l,h}) * w_{l,h} ),  l = l10, l12, l20
//   E       = max_l S_l  or  mean_l S_l
//
// Per request row this is a [N x 128] x [128 x 192] contraction (3 layers x
// 64 heads), 49152 flop per 132-byte chunk, on the 16x16x32 f16 MFMA.
// Exact-algebra choices that keep it within the fp64 result:
//   - the e4m3 codes are converted exactly to f16 (every finite e4m3 value
//     is an f16 value); the fp32 scale is applied to the fp32 head sum, not
//     folded into the operand: relu(s x) = |s| relu(sign(s) x), and a
//     negative scale flips the decoded operand's signs instead;
//   - q is rounded once to f16 (11-bit significand).
#include "fm_internal.h"

namespace fm {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// MFMA 16x16x32 f16 operand layout: lane l supplies A[l%16][8(l/16) + e] and
// B[8(l/16) + e][l%16], e = 0..7, and receives C[4(l/16) + r][l%16].
// A = queries (rows = 16 heads of a head tile), B = keys (columns = 16
// chunks).  For k-step t (t = 0..3) lane l's eight k slots are the dims
// 32(l/16) + 8t + e, so each lane reads one contiguous 32-byte run of its
// chunk's codes.  Fragment f = (layer * 4 + head_tile) * 4 + t.
__global__ __launch_bounds__(256) void pack_q_kernel(const float* q, int B, f16x8* qpack) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= B * kQFrags * 64) return;
  const int lane = gid & 63;
  const int f = (gid >> 6) % kQFrags;
  const int b = gid / (64 * kQFrags);
  const int t = f & 3;
  const int mt = (f >> 2) & 3;
  const int layer = f >> 4;
  const int head = 16 * mt + (lane & 15);
  const int d0 = 32 * (lane >> 4) + 8 * t;
  const float* src = q + (((size_t)layer * B + b) * kHeads + head) * kHeadDim + d0;
  f16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (_Float16)src[e];
  qpack[gid] = v;
}

__device__ inline f16x8 decode8(uint32_t lo, uint32_t hi) {
  // four 2-code conversions; scale 1.0 leaves the value unchanged
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Sum over the four lane groups {l, l^16, l^32, l^48} (every lane gets it).
__device__ inline float sum4groups(float v) {
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

__device__ inline float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// grid = (ceil(N / (4 * CPW)), B), block = 256: wave w of block x scores
// chunks [(4x + w) CPW, +CPW) of row blockIdx.y, 16 chunks per step.
template <int CPW>
__global__ __launch_bounds__(256) void score_kernel(const f16x8* __restrict__ qpack, const float* __restrict__ w,
                                                    const uint8_t* __restrict__ comp_k, int B, int64_t N,
                                                    const int32_t* __restrict__ valid_n, int mode,
                                                    float* __restrict__ scores, float* __restrict__ per_layer) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t start = ((int64_t)blockIdx.x * 4 + wave) * CPW;
  if (start >= N) return;
  const int64_t end = start + CPW < N ? start + CPW : N;
  int64_t vn = N;
  if (valid_n) {
    const int64_t v = valid_n[b];
    vn = v < 0 ? 0 : (v > N ? N : v);
  }
  const int64_t vend = end < vn ? end : vn;

  // Tail at or beyond valid_n: -inf, bytes not read.
  {
    const float ninf = -__builtin_huge_valf();
    for (int64_t n = (start > vn ? start : vn) + lane; n < end; n += 64) {
      scores[(size_t)b * N + n] = ninf;
      if (per_layer)
        for (int l = 0; l < kLayers; ++l) per_layer[((size_t)l * B + b) * N + n] = ninf;
    }
  }
  if (start >= vend) return;

  const int c = lane & 15;
  const int g = lane >> 4;

  f16x8 qf[kLayers][4][4];
  {
    const f16x8* qp = qpack + (size_t)b * kQFrags * 64 + lane;
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) qf[l][mt][t] = qp[((l * 4 + mt) * 4 + t) * 64];
  }
  // w of the heads this lane's accumulators hold: 16 mt + 4 g + r.
  f32x4 wv[kLayers][4];
#pragma unroll
  for (int l = 0; l < kLayers; ++l)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      wv[l][mt] = *(const f32x4*)(w + ((size_t)l * B + b) * kHeads + 16 * mt + 4 * g);

  const uint8_t* row = comp_k + (size_t)b * N * kRecord;
  for (int64_t n0 = start; n0 < vend; n0 += 16) {
    const int64_t n = n0 + c;
    const bool valid = n < vend;
    u32x8 raw = {0, 0, 0, 0, 0, 0, 0, 0};
    float s = 0.f;
    if (valid) {
      const uint8_t* rp = row + (size_t)n * kRecord;
      const u32x4 r0 = *(const u32x4_a4*)(rp + 32 * g);
      const u32x4 r1 = *(const u32x4_a4*)(rp + 32 * g + 16);
      raw = u32x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
      s = *(const float*)(rp + kHeadDim);
    }
    f16x8 kf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) kf[t] = decode8(raw[2 * t], raw[2 * t + 1]);
    // A negative scale: relu(s x) = |s| relu(-x); flip the operand's signs.
    if (__builtin_amdgcn_read_exec() & __ballot(s < 0.f)) {
      if (s < 0.f) {
#pragma unroll
        for (int t = 0; t < 4; ++t) kf[t] = -kf[t];
      }
    }

    f32x4 acc[kLayers][4];
#pragma unroll
    for (int l = 0; l < kLayers; ++l)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[l][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int l = 0; l < kLayers; ++l)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[l][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qf[l][mt][t], kf[t], acc[l][mt], 0, 0, 0);

    const float as = fabsf(s);
    float S[kLayers];
#pragma unroll
    for (int l = 0; l < kLayers; ++l) {
      float p = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p = fmaf(fmaxf(acc[l][mt][r], 0.f), wv[l][mt][r], p);
      p = sum4groups(p);
      S[l] = sigmoidf_(as * p);
    }
    const float E = mode == FM_ENSEMBLE_MAX ? fmaxf(fmaxf(S[0], S[1]), S[2]) : (S[0] + S[1] + S[2]) / 3.0f;
    if (valid) {
      if (g == 0) scores[(size_t)b * N + n] = E;
      if (per_layer && g < kLayers) {
        const float v = g == 0 ? S[0] : (g == 1 ? S[1] : S[2]);
        per_layer[((size_t)g * B + b) * N + n] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_score(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B, int64_t N,
                        const int32_t* valid_n, int mode, float* scores, float* per_layer, hipStream_t stream) {
  f16x8* qpack = (f16x8*)ws.qpack;
  {
    const int total = B * kQFrags * 64;
    hipLaunchKernelGGL(pack_q_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, q, B, qpack);
  }
  constexpr int kCPW = 1024;
  const int64_t per_block = 4 * (int64_t)kCPW;
  dim3 grid((unsigned)((N + per_block - 1) / per_block), (unsigned)B);
  hipLaunchKernelGGL((score_kernel<kCPW>), grid, dim3(256), 0, stream, (const f16x8*)qpack, w, comp_k, B, N, valid_n,
                     mode, scores, per_layer);
  return hipGetLastError();
}

}  // namespace fm
