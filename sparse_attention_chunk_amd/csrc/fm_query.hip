// Query and weight branches of the Memory-Indexer (FlashMemory DS-V4
// Retriever README, "Architecture"):
//   a      = wq_a hidden                      (Q_LORA_RANK)
//   a_hat  = RMSNorm(a) * q_norm_weight       (eps inside the root)
//   q_lin  = wq_b a_hat, viewed [N_HEADS][HEAD_DIM] head-major
//   q      = Hadamard(RoPE_YaRN(q_lin))       (RoPE on the last 64 dims)
//   w      = weights_proj hidden * HEAD_DIM^-0.5 N_HEADS^-0.5
//
// The projections are skinny fp32 GEMMs (B <= a few dozen rows against up
// to 8192 weight rows), bound by streaming the fp32 weights from HBM.  They
// run on the fp32 MFMA (v_mfma_f32_16x16x4_f32): the vector unit without
// packed fp32 would need ~2x the issue slots for the same flops.
#include "fm_internal.h"

#include <cmath>

namespace fm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

struct ProjArgs {
  const float* w0[kLayers];  // rows [0, rows0) of the stacked weight, per layer
  const float* w1[kLayers];  // rows [rows0, rows0 + rows1), per layer (may be null when rows1 == 0)
  const float* x;            // activations: x + layer * x_layer_stride + b * K
  float* out;                // out[split][layer][b][rows0 + rows1]
  long x_layer_stride;
  int rows0, rows1, K, k_split, B;
};

// C[b][o] = sum_k x[b][k] W[o][k] on 16x16x4 fp32 MFMA tiles.  A wave owns
// OT column tiles (16 outputs each) x BT row tiles (16 batch rows each) over
// one K slice; a 256-thread block holds 4 waves on consecutive column groups.
//
// MFMA operand layout (16x16x4 f32): lane l supplies A[l%16][l/16] and
// B[l/16][l%16] and receives C[4(l/16)+r][l%16], r = 0..3.  Each lane loads
// 4 consecutive k of one row (a float4); MFMA e of a 16-k step takes element
// e, so the four MFMAs of a step cover the 16 k exactly once.
template <int OT, int BT>
__global__ __launch_bounds__(256) void proj_kernel(ProjArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rows = p.rows0 + p.rows1;
  const int o_base = (blockIdx.x * 4 + wave) * 16 * OT;
  if (o_base >= rows) return;
  const int layer = blockIdx.y / p.k_split;
  const int split = blockIdx.y % p.k_split;
  const int k_len = p.K / p.k_split;
  const int k_begin = split * k_len;
  const int b_base = blockIdx.z * 16 * BT;
  const int i = lane & 15;
  const int g = lane >> 4;

  const float* wrow[OT];
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    const int o = o_base + 16 * ot + i;
    wrow[ot] = o < p.rows0 ? p.w0[layer] + (size_t)o * p.K
                           : (o < rows ? p.w1[layer] + (size_t)(o - p.rows0) * p.K : nullptr);
  }
  const float* xrow[BT];
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) {
    const int b = b_base + 16 * bt + i;
    xrow[bt] = b < p.B ? p.x + layer * p.x_layer_stride + (size_t)b * p.K : nullptr;
  }

  f32x4 acc[OT][BT];
#pragma unroll
  for (int ot = 0; ot < OT; ++ot)
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) acc[ot][bt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int k = k_begin + 4 * g; k < k_begin + k_len; k += 16) {
    f32x4 wv[OT], xv[BT];
#pragma unroll
    for (int ot = 0; ot < OT; ++ot) wv[ot] = wrow[ot] ? *(const f32x4*)(wrow[ot] + k) : zero;
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) xv[bt] = xrow[bt] ? *(const f32x4*)(xrow[bt] + k) : zero;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int ot = 0; ot < OT; ++ot)
#pragma unroll
        for (int bt = 0; bt < BT; ++bt)
          acc[ot][bt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[bt][e], wv[ot][e], acc[ot][bt], 0, 0, 0);
  }

  // C rows are batch rows, C columns outputs: lane l holds b = 4(l/16)+r, o = l%16.
#pragma unroll
  for (int ot = 0; ot < OT; ++ot) {
    const int o = o_base + 16 * ot + i;
    if (o >= rows) continue;
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int b = b_base + 16 * bt + 4 * g + r;
        if (b < p.B) p.out[(((size_t)split * kLayers + layer) * p.B + b) * rows + o] = acc[ot][bt][r];
      }
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// One wave per (layer, row): adds the K-slice partials in slice order, then
// RMSNorm (a / sqrt(mean(a^2) + eps) * gain) of the Q_LORA_RANK vector, and
// finishes the weight branch (weights_proj rows times weight_scale).
struct GainPtrs {
  const float* g[kLayers];
};

__global__ __launch_bounds__(64) void rmsnorm_kernel(const float* part, GainPtrs gains, int B, float eps,
                                                     float w_scale, float* a_hat, float* w_out) {
  const int layer = blockIdx.x / B;
  const int b = blockIdx.x % B;
  const int lane = threadIdx.x;
  const size_t split_stride = (size_t)kLayers * B * kProj1Out;
  const float* src = part + ((size_t)layer * B + b) * kProj1Out;
  float a[kQLora / 64];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kQLora / 64; ++i) {
    const int o = lane + 64 * i;
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < kSplitK1; ++s) v += src[s * split_stride + o];
    a[i] = v;
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss * (1.0f / kQLora) + eps);
  const float* gain = gains.g[layer];
  float* dst = a_hat + ((size_t)layer * B + b) * kQLora;
#pragma unroll
  for (int i = 0; i < kQLora / 64; ++i) {
    const int o = lane + 64 * i;
    dst[o] = a[i] * rs * gain[o];
  }
  float wv = 0.f;
#pragma unroll
  for (int s = 0; s < kSplitK1; ++s) wv += src[s * split_stride + kQLora + lane];
  w_out[((size_t)layer * B + b) * kHeads + lane] = wv * w_scale;
}

// One block per (layer, row), 4 waves of 16 heads.  Lane l holds dims 2l and
// 2l+1 of a head.  RoPE: lanes 32..63 hold the rotated dims 64..127, pair
// j = l - 32 is turned counter-clockwise by pos * freq[j]; the angle and its
// cosine/sine are formed in double precision (positions reach 2^20 and the
// first frequency is 1 rad/token), the rotation itself in fp32.  Then the
// 128-point Walsh-Hadamard butterfly in Sylvester order, scaled by 128^-0.5.
__global__ __launch_bounds__(256) void rope_hadamard_kernel(const float* q_lin, const int64_t* positions,
                                                            const double* freq, int B, float* q_out) {
  const int layer = blockIdx.x / B;
  const int b = blockIdx.x % B;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float cs = 1.f, sn = 0.f;
  if (lane >= 32) {
    const double phi = (double)positions[b] * freq[lane - 32];
    cs = (float)cos(phi);
    sn = (float)sin(phi);
  }
  const float inv_sqrt = 0.08838834764831845f;  // 128^-0.5
  const size_t base = ((size_t)layer * B + b) * kHeads * kHeadDim;
  for (int hh = 0; hh < 16; ++hh) {
    const int h = wave * 16 + hh;
    const float2 v = *(const float2*)(q_lin + base + (size_t)h * kHeadDim + 2 * lane);
    float x = v.x, y = v.y;
    if (lane >= 32) {
      const float rx = x * cs - y * sn;
      const float ry = x * sn + y * cs;
      x = rx;
      y = ry;
    }
    float a0 = x + y;
    float a1 = x - y;
#pragma unroll
    for (int m = 1; m <= 32; m <<= 1) {
      const float p0 = __shfl_xor(a0, m, 64);
      const float p1 = __shfl_xor(a1, m, 64);
      if (lane & m) {
        a0 = p0 - a0;
        a1 = p1 - a1;
      } else {
        a0 = a0 + p0;
        a1 = a1 + p1;
      }
    }
    *(float2*)(q_out + base + (size_t)h * kHeadDim + 2 * lane) = make_float2(a0 * inv_sqrt, a1 * inv_sqrt);
  }
}

}  // namespace

hipError_t launch_prepare_query(const fm_config& cfg, const fm_weights& wts, const Workspace& ws, int max_batch,
                                const float* hidden, const int64_t* positions, int B, float* q_out, float* w_out,
                                hipStream_t stream) {
  (void)max_batch;
  constexpr int kBT = 2;  // 32 batch rows per wave; more rows go to grid.z
  const int b_groups = (B + 16 * kBT - 1) / (16 * kBT);

  // wq_a | weights_proj, split over K.
  {
    ProjArgs p{};
    for (int l = 0; l < kLayers; ++l) {
      p.w0[l] = wts.wq_a[l];
      p.w1[l] = wts.w_proj[l];
    }
    p.x = hidden;
    p.x_layer_stride = 0;
    p.out = ws.proj1_part;
    p.rows0 = kQLora;
    p.rows1 = kHeads;
    p.K = kHidden;
    p.k_split = kSplitK1;
    p.B = B;
    constexpr int kOT = 1;
    const int col_groups = (kProj1Out + 16 * kOT - 1) / (16 * kOT);
    dim3 grid((col_groups + 3) / 4, kLayers * kSplitK1, b_groups);
    hipLaunchKernelGGL((proj_kernel<kOT, kBT>), grid, dim3(256), 0, stream, p);
  }
  // RMSNorm + weight-branch finish.
  {
    GainPtrs gp{};
    for (int l = 0; l < kLayers; ++l) gp.g[l] = wts.q_norm[l];
    const float w_scale = (float)(1.0 / std::sqrt((double)cfg.head_dim * (double)cfg.n_heads));
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(kLayers * B), dim3(64), 0, stream, ws.proj1_part, gp, B, cfg.rms_eps,
                       w_scale, ws.a_hat, w_out);
  }
  // wq_b.
  {
    ProjArgs p{};
    for (int l = 0; l < kLayers; ++l) {
      p.w0[l] = wts.wq_b[l];
      p.w1[l] = nullptr;
    }
    p.x = ws.a_hat;
    p.x_layer_stride = (long)B * kQLora;
    p.out = ws.q_lin;
    p.rows0 = kHeads * kHeadDim;
    p.rows1 = 0;
    p.K = kQLora;
    p.k_split = 1;
    p.B = B;
    constexpr int kOT = 2;
    const int col_groups = (kHeads * kHeadDim + 16 * kOT - 1) / (16 * kOT);
    dim3 grid((col_groups + 3) / 4, kLayers, b_groups);
    hipLaunchKernelGGL((proj_kernel<kOT, kBT>), grid, dim3(256), 0, stream, p);
  }
  // RoPE (YaRN) + normalized Hadamard.
  hipLaunchKernelGGL(rope_hadamard_kernel, dim3(kLayers * B), dim3(256), 0, stream, ws.q_lin, positions,
                     ws.rope_freq, B, q_out);
  return hipGetLastError();
}

}  // namespace fm
