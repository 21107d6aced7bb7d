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

struct ProjArgs {
  const float* w0[kLayers];  // rows [0, rows0) of the stacked weight, per layer
  const float* w1[kLayers];  // rows [rows0, rows0 + rows1), per layer (may be null when rows1 == 0)
  const float* x;            // activations: x + layer * x_layer_stride + b * K
  float* out;                // out[split][layer][b][rows0 + rows1]
  long x_layer_stride;
  int rows0, rows1, K, k_split, B;
};

// C[b][o] = sum_k x[b][k] W[o][k] on 16x16x4 fp32 MFMA tiles.  A block of
// 4 waves owns 4 consecutive column tiles (64 outputs) x 32 batch rows over
// one K slice, walked in kKChunk-wide chunks.  Each wave streams its own 16
// weight rows from HBM, the weights of chunk c+1 requested before chunk c is
// multiplied (two register buffers), so the weight stream and the MFMAs
// overlap inside every wave.  The 32 activation rows of each chunk are
// staged in LDS (two buffers) and shared by the 4 waves.
//
// MFMA operand layout (16x16x4 f32): lane l supplies A[l%16][l/16] and
// B[l/16][l%16] and receives C[4(l/16)+r][l%16], r = 0..3.  Each lane loads
// 4 consecutive k of one row (a float4); MFMA e of a 16-k step takes element
// e, so the four MFMAs of a step cover the 16 k exactly once.
constexpr int kKChunk = 256;
constexpr int kXStride = kKChunk + 4;  // padded LDS row (floats): rows start in different banks
constexpr int kWSteps = kKChunk / 16;  // float4 weight loads per lane per chunk
constexpr int kStage = kProjRowsPerWave * kKChunk / 4 / 256;  // float4 activation loads per thread per chunk

constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

// Per-wave operand descriptors: reads past a descriptor's range return
// zeros, which stands in for weight rows past the last output and batch
// rows past B without a branch.
struct ProjLane {
  __amdgpu_buffer_rsrc_t w;  // this wave's 16 weight rows (fewer at the end)
  __amdgpu_buffer_rsrc_t x;  // activation rows [0, B) of the layer
  uint32_t w_off;            // byte offset of lane's row, k = 4 g
  int K, b_base;
};

__device__ __forceinline__ void proj_load_w(const ProjLane& pl, int kc, f32x4 (&wv)[kWSteps]) {
#pragma unroll
  for (int u = 0; u < kWSteps; ++u)
    wv[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pl.w, pl.w_off + 4u * (kc + 16 * u), 0, 0));
}

// Activation rows b_base .. b_base + 32 of chunk kc, to registers.
__device__ __forceinline__ void proj_load_x(const ProjLane& pl, int kc, f32x4 (&xr)[kStage]) {
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int idx = threadIdx.x + 256 * j;
    const uint32_t off = 4u * ((uint32_t)(pl.b_base + idx / (kKChunk / 4)) * pl.K + kc + 4 * (idx % (kKChunk / 4)));
    xr[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pl.x, off, 0, 0));
  }
}

__device__ __forceinline__ void proj_store_x(const f32x4 (&xr)[kStage], float* xs) {
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int idx = threadIdx.x + 256 * j;
    *(f32x4*)(xs + (idx / (kKChunk / 4)) * kXStride + 4 * (idx % (kKChunk / 4))) = xr[j];
  }
}

template <int BT>
__device__ __forceinline__ void proj_mfma(const f32x4 (&wv)[kWSteps], const float* xs, int i, int g,
                                          f32x4 (&acc)[BT]) {
#pragma unroll
  for (int u = 0; u < kWSteps; ++u) {
    f32x4 xv[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) xv[bt] = *(const f32x4*)(xs + (16 * bt + i) * kXStride + 4 * g + 16 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int bt = 0; bt < BT; ++bt) acc[bt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[bt][e], wv[u][e], acc[bt], 0, 0, 0);
  }
}

// Workgroup barrier ordering LDS only: weight and activation loads of the
// next chunk stay in flight across it (a full barrier would drain them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CHUNKS>
__global__ __launch_bounds__(256) void proj_kernel(ProjArgs p) {
  constexpr int BT = kProjRowsPerWave / 16;
  __shared__ f32x4 xs4[kProjRowsPerWave * kXStride / 4];
  float* xs = (float*)xs4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = p.rows0 + p.rows1;
  const int o_base = (blockIdx.x * 4 + wave) * 16;
  const int layer = blockIdx.y / p.k_split;
  const int split = blockIdx.y % p.k_split;
  const int k_begin = split * (CHUNKS * kKChunk);
  const int i = lane & 15;

  const int g = lane >> 4;
  ProjLane pl;
  {
    // The wave's 16 rows lie in one of the two stacked weights (rows0 is a
    // multiple of 16); past the last row the range is empty.
    const bool second = o_base >= p.rows0;
    const int r0 = second ? o_base - p.rows0 : o_base;
    const int avail = (second ? p.rows1 : p.rows0) - r0;
    const int nrows = avail < 0 ? 0 : (avail > 16 ? 16 : avail);
    // Static indices keep the pointers in scalar registers.
    const float* w0 = layer == 0 ? p.w0[0] : (layer == 1 ? p.w0[1] : p.w0[2]);
    const float* w1 = layer == 0 ? p.w1[0] : (layer == 1 ? p.w1[1] : p.w1[2]);
    const float* wbase = (second ? w1 : w0) + (size_t)r0 * p.K;  // never read when nrows is 0
    // The values are wave-uniform; readfirstlane keeps the descriptor in
    // scalar registers (a vector-register descriptor costs a loop per load).
    const uint64_t wa = (uint64_t)(uintptr_t)wbase;
    const uint64_t wu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(wa >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)wa);
    pl.w = __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)wu, 0,
                                             __builtin_amdgcn_readfirstlane(nrows * p.K * 4), kBufferWord3);
    pl.w_off = 4u * ((uint32_t)i * p.K + 4 * g);
    pl.x = __builtin_amdgcn_make_buffer_rsrc((void*)(p.x + layer * p.x_layer_stride), 0, p.B * p.K * 4, kBufferWord3);
    pl.K = p.K;
    pl.b_base = blockIdx.z * kProjRowsPerWave;
  }
  const int o = o_base + i;

  f32x4 acc[BT];
#pragma unroll
  for (int bt = 0; bt < BT; ++bt) acc[bt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Straight-line over the chunks (two static weight buffers): the weights
  // and activations of chunk c+1 are requested before chunk c is
  // multiplied; the activations reach LDS after the barrier that ends every
  // wave's use of chunk c.
  f32x4 wbuf[2][kWSteps], xr[kStage];
  proj_load_w(pl, k_begin, wbuf[0]);
  proj_load_x(pl, k_begin, xr);
  proj_store_x(xr, xs);
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    if (c + 1 < CHUNKS) {
      proj_load_w(pl, k_begin + (c + 1) * kKChunk, wbuf[(c + 1) & 1]);
      proj_load_x(pl, k_begin + (c + 1) * kKChunk, xr);
    }
    lds_barrier();
    proj_mfma<BT>(wbuf[c & 1], xs, i, g, acc);
    if (c + 1 < CHUNKS) {
      lds_barrier();
      proj_store_x(xr, xs);
    }
  }

  // C rows are batch rows, C columns outputs: lane l holds b = 4(l/16)+r, o = l%16.
  if (o < rows) {
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int b = pl.b_base + 16 * bt + 4 * g + r;
        if (b < p.B) p.out[(((size_t)split * kLayers + layer) * p.B + b) * rows + o] = acc[bt][r];
      }
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
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
                                                      float* rope_cs, float* a_hat, float* w_out) {
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
  float* dst = a_hat + ((size_t)layer * B + b) * kQLora;
  const f32x4 gv = {gain[4 * t], gain[4 * t + 1], gain[4 * t + 2], gain[4 * t + 3]};
  *(f32x4*)(dst + 4 * t) = a * rs * gv;
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

// One wave per (layer, row, head), 4 heads per block.  Lane l holds dims 2l
// and 2l+1 of the head (the wq_b K-slice partials added in slice order).
// RoPE: lanes 32..63 hold the rotated dims 64..127; pair j = l - 32 is
// turned counter-clockwise by pos * freq[j] (cosine and sine from the
// RMSNorm kernel), the rotation in fp32.  Then the 128-point Walsh-Hadamard
// butterfly in Sylvester order, scaled by 128^-0.5.
__global__ __launch_bounds__(256) void rope_hadamard_kernel(const float* q_lin, int splits, const float* rope_cs, int B,
                                                            float* q_out) {
  const int lane = threadIdx.x & 63;
  const int gh = blockIdx.x * 4 + (threadIdx.x >> 6);  // (layer * B + b) * 64 + h
  const int h = gh % kHeads;
  const int lb = gh / kHeads;
  const int b = lb % B;
  const size_t off = (size_t)lb * kHeads * kHeadDim + (size_t)h * kHeadDim + 2 * lane;
  const size_t split_stride = (size_t)kLayers * B * kHeads * kHeadDim;
  float x = 0.f, y = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float2 v = *(const float2*)(q_lin + s * split_stride + off);
    x += v.x;
    y += v.y;
  }
  if (lane >= 32) {
    const float2 c = *(const float2*)(rope_cs + ((size_t)b * (kRopeDim / 2) + (lane - 32)) * 2);
    const float rx = x * c.x - y * c.y;
    const float ry = x * c.y + y * c.x;
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
  const float inv_sqrt = 0.08838834764831845f;  // 128^-0.5
  *(float2*)(q_out + off) = make_float2(a0 * inv_sqrt, a1 * inv_sqrt);
}

// K slice = 4, 8 or 16 chunks of 256 (the split counts keep it there).
void launch_proj(const ProjArgs& p, dim3 grid, hipStream_t stream) {
  const int chunks = p.K / p.k_split / kKChunk;
  auto kern = chunks == 4 ? proj_kernel<4> : (chunks == 8 ? proj_kernel<8> : proj_kernel<16>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, p);
}

}  // namespace

hipError_t launch_prepare_query(const fm_config& cfg, const fm_weights& wts, const Workspace& ws, int max_batch,
                                const float* hidden, const int64_t* positions, int B, float* q_out, float* w_out,
                                hipStream_t stream) {
  (void)max_batch;
  const int row_groups = proj_row_groups(B);
  const int s1 = proj1_splits(B);
  const int s2 = proj2_splits(B);

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
    p.k_split = s1;
    p.B = B;
    const int col_tiles = (kProj1Out + 15) / 16;
    dim3 grid((col_tiles + 3) / 4, kLayers * s1, row_groups);
    launch_proj(p, grid, stream);
  }
  // RMSNorm + weight-branch finish + RoPE angles.
  {
    GainPtrs gp{};
    for (int l = 0; l < kLayers; ++l) gp.g[l] = wts.q_norm[l];
    const float w_scale = (float)(1.0 / std::sqrt((double)cfg.head_dim * (double)cfg.n_heads));
    auto kern = s1 == 4 ? rmsnorm_kernel<4> : (s1 == 2 ? rmsnorm_kernel<2> : rmsnorm_kernel<1>);
    hipLaunchKernelGGL(kern, dim3(kLayers * B), dim3(256), 0, stream, ws.proj1_part, gp, B, cfg.rms_eps, w_scale,
                       positions, ws.rope_freq, ws.rope_cs, ws.a_hat, w_out);
  }
  // wq_b, split over K.
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
    p.k_split = s2;
    p.B = B;
    const int col_tiles = kHeads * kHeadDim / 16;
    dim3 grid((col_tiles + 3) / 4, kLayers * s2, row_groups);
    launch_proj(p, grid, stream);
  }
  // Split-K sum, RoPE (YaRN) + normalized Hadamard.
  hipLaunchKernelGGL(rope_hadamard_kernel, dim3(kLayers * B * kHeads / 4), dim3(256), 0, stream, ws.q_lin, s2,
                     ws.rope_cs, B, q_out);
  return hipGetLastError();
}

}  // namespace fm
