// C ABI of libfm (include/fm.h): argument checks, the context and its
// workspace, and dispatch to the kernel launchers.  Every check runs before
// anything is enqueued, so a failing call leaves the stream untouched.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "fm_internal.h"

namespace {

// The calling thread's last error message (a fixed buffer: no call
// allocates, on any path).
thread_local char g_err[512];

fm_status fail(fm_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_err() { g_err[0] = 0; }

fm_status hip_fail(hipError_t e, const char* what) {
  return fail(FM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Frequencies theta'_j, j < rope_dim/2, in double precision (README
// "Architecture": RoPE with YaRN, base 160000, on the last rope_dim dims).
// theta_j = base^(-2j/d).  For yarn_factor s > 1 the frequencies blend
// linearly in j from theta_j (j <= lo) to theta_j / s (j >= hi), where lo and
// hi are the indices whose wavelengths complete beta_fast and beta_slow
// turns over the original context: j(r) = d ln(L0 / (2 pi r)) / (2 ln base),
// lo = floor(j(beta_fast)), hi = ceil(j(beta_slow)), clamped to [0, d-1];
// equal bounds are separated by 0.001.
void rope_frequencies(const fm_config& c, double* out) {
  const int d = c.rope_dim;
  const int half = d / 2;
  const double pi = 3.14159265358979323846;
  double lo = 0, hi = 1;
  const bool yarn = c.yarn_factor != 1.0;
  if (yarn) {
    auto jr = [&](double turns) {
      return d * std::log((double)c.yarn_orig_ctx / (turns * 2.0 * pi)) / (2.0 * std::log(c.rope_base));
    };
    lo = std::floor(jr(c.yarn_beta_fast));
    hi = std::ceil(jr(c.yarn_beta_slow));
    if (lo < 0) lo = 0;
    if (hi > d - 1) hi = d - 1;
    if (lo == hi) hi += 0.001;
  }
  for (int j = 0; j < half; ++j) {
    const double theta = std::pow(c.rope_base, -2.0 * j / d);
    if (!yarn) {
      out[j] = theta;
      continue;
    }
    double ramp = (j - lo) / (hi - lo);
    ramp = ramp < 0 ? 0 : (ramp > 1 ? 1 : ramp);
    out[j] = theta * (1.0 - ramp) + (theta / c.yarn_factor) * ramp;
  }
}

fm_status check_ctx(fm_ctx* ctx) {
  if (!ctx) return fail(FM_EINVAL, "null context");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != ctx->device) return fail(FM_EINVAL, "context belongs to device %d but device %d is current", ctx->device, dev);
  return FM_OK;
}

fm_status check_shape(const fm_ctx* ctx, int32_t B, int64_t N, bool with_n) {
  if (B < 0 || B > ctx->max_batch) return fail(FM_EINVAL, "B = %d outside [0, %d]", B, ctx->max_batch);
  if (with_n && (N < 0 || N > ctx->max_n))
    return fail(FM_EINVAL, "N = %lld outside [0, %lld]", (long long)N, (long long)ctx->max_n);
  return FM_OK;
}

}  // namespace

// Device scratch of fm_select_topk_static, for callers that cannot allocate:
// the top-K scan's tile words.  Every GPU the library runs on holds its own
// copy until the process ends; host code reaches it only through the
// address hipGetSymbolAddress gives on that device (the array's name is a
// host-side stand-in, not a device address).
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device `dev`, looked up on
// the first call there and kept.
hipError_t static_scratch(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

void fm_config_default(fm_config* cfg) {
  if (!cfg) return;
  cfg->n_layers = 3;
  cfg->hidden = 4096;
  cfg->q_lora_rank = 1024;
  cfg->n_heads = 64;
  cfg->head_dim = 128;
  cfg->rope_dim = 64;
  cfg->rms_eps = 1e-6f;
  cfg->rope_base = 160000.0;
  cfg->yarn_factor = 1.0;
  cfg->yarn_orig_ctx = 65536;
  cfg->yarn_beta_fast = 32.0;
  cfg->yarn_beta_slow = 1.0;
}

const char* fm_last_error(void) { return g_err; }

fm_status fm_create(const fm_config* cfg, const fm_weights* weights, int32_t max_batch, int64_t max_n,
                    fm_ctx** out) {
  clear_err();
  if (!cfg || !weights || !out) return fail(FM_EINVAL, "null argument to fm_create");
  *out = nullptr;
  using namespace fm;
  if (cfg->n_layers != kLayers || cfg->hidden != kHidden || cfg->q_lora_rank != kQLora || cfg->n_heads != kHeads ||
      cfg->head_dim != kHeadDim || cfg->rope_dim != kRopeDim)
    return fail(FM_EUNSUPPORTED,
                "compiled for n_layers 3, hidden 4096, q_lora_rank 1024, n_heads 64, head_dim 128, rope_dim 64");
  if (!(cfg->rms_eps >= 0.f) || !std::isfinite(cfg->rms_eps)) return fail(FM_EINVAL, "rms_eps must be finite and >= 0");
  if (!(cfg->rope_base > 1.0) || !std::isfinite(cfg->rope_base)) return fail(FM_EINVAL, "rope_base must be > 1");
  if (!(cfg->yarn_factor >= 1.0) || !std::isfinite(cfg->yarn_factor)) return fail(FM_EINVAL, "yarn_factor must be >= 1");
  if (cfg->yarn_factor != 1.0 && (cfg->yarn_orig_ctx <= 0 || !(cfg->yarn_beta_fast > 0) || !(cfg->yarn_beta_slow > 0)))
    return fail(FM_EINVAL, "YaRN needs yarn_orig_ctx > 0 and positive betas");
  if (max_batch < 1 || max_batch > 4096) return fail(FM_EINVAL, "max_batch = %d outside [1, 4096]", max_batch);
  if (max_n < 1 || max_n > (int64_t(1) << 26)) return fail(FM_EINVAL, "max_n outside [1, 2^26]");
  for (int l = 0; l < kLayers; ++l) {
    if (!weights->wq_a[l] || !weights->q_norm[l] || !weights->wq_b[l] || !weights->w_proj[l])
      return fail(FM_EINVAL, "null weight pointer (layer %d)", l);
    if (!aligned(weights->wq_a[l], 16) || !aligned(weights->wq_b[l], 16) || !aligned(weights->w_proj[l], 16) ||
        !aligned(weights->q_norm[l], 4))
      return fail(FM_EINVAL, "weights must be 16-byte aligned (q_norm 4-byte)");
  }

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
  if (cus < 1 || cus > kMaxScoreBlocks) return fail(FM_EUNSUPPORTED, "device reports %d compute units", cus);

  // One allocation, each buffer 256-byte aligned.  The split-K partial
  // buffer holds splits(B) * B rows, largest at B = max_batch or at the
  // largest B of the most-split row-group count.
  const size_t mb = (size_t)max_batch;
  size_t p1_rows = 0;
  for (int g = 1; g <= proj_row_groups(max_batch); ++g) {
    const int b = g * kProjRowsPerWave < max_batch ? g * kProjRowsPerWave : max_batch;
    p1_rows = std::max(p1_rows, (size_t)proj1_splits(b) * b);
  }
  enum {
    kW1, kW1Inv, kW2, kW2Inv, kGain, kPart1, kAHatHi, kAHatLo, kAHatInv, kFreq, kCosSin, kQPack, kQPack8, kW8, kRowTiles, kWaveRow,
    kSubKeys, kSubTiles, kResCount, kResBits, kTileInfo, kNumBuffers
  };
  size_t sizes[kNumBuffers];
  sizes[kW1] = (size_t)4 * kLayers * kProj1Out * kHidden;  // two f16 parts per weight
  sizes[kW1Inv] = sizeof(float) * kLayers * kProj1Out;
  sizes[kW2] = (size_t)4 * kLayers * kHeads * kHeadDim * kQLora;
  sizes[kW2Inv] = sizeof(float) * kLayers * kHeads * kHeadDim;
  sizes[kGain] = sizeof(float) * kLayers * kQLora;
  sizes[kPart1] = sizeof(float) * kLayers * p1_rows * kProj1Out;
  sizes[kAHatHi] = sizeof(_Float16) * kLayers * mb * kQLora;
  sizes[kAHatLo] = sizeof(_Float16) * kLayers * mb * kQLora;
  sizes[kAHatInv] = sizeof(float) * kLayers * mb * (kQLora / 128);
  sizes[kFreq] = sizeof(double) * (kRopeDim / 2);
  sizes[kCosSin] = sizeof(float) * mb * kRopeDim;
  sizes[kQPack] = (size_t)16 * kQFrags * 64 * mb;        // f16x8 per lane
  sizes[kQPack8] = (size_t)32 * kQ8Frags * 64 * mb;      // 32 e4m3 bytes per lane
  sizes[kW8] = sizeof(float) * kW8Row * mb;
  sizes[kRowTiles] = sizeof(int64_t) * (mb + 1);
  sizes[kWaveRow] = sizeof(int32_t) * 4 * (size_t)cus;
  sizes[kSubKeys] = sizeof(uint32_t) * mb * kSubFastCap;
  sizes[kSubTiles] = sizeof(uint2) * mb * (kSubFastCap / 16);
  sizes[kResCount] = 3 * sizeof(uint32_t) * mb * (size_t)((max_n + kResSlice - 1) / kResSlice);
  sizes[kResBits] = sizeof(unsigned long long) * mb * (size_t)((max_n + kResSlice - 1) / kResSlice) * (kResSlice / 16);
  sizes[kTileInfo] = sizeof(uint2) * mb * (size_t)fm::tile_info_stride(max_n);
  size_t offs[kNumBuffers];
  size_t total = 0;
  for (int i = 0; i < kNumBuffers; ++i) {
    offs[i] = total;
    total += (sizes[i] + 255) & ~(size_t)255;
  }
  void* base = nullptr;
  e = hipMalloc(&base, total);
  if (e != hipSuccess) return fail(FM_ENOMEM, "workspace of %zu bytes: %s", total, hipGetErrorString(e));

  fm_ctx* ctx = new fm_ctx();
  ctx->device = dev;
  ctx->cfg = *cfg;
  ctx->weights = *weights;
  ctx->max_batch = max_batch;
  ctx->max_n = max_n;
  ctx->ws_base = base;
  ctx->ws_bytes = total;
  char* p = (char*)base;
  ctx->ws.w1 = (_Float16*)(p + offs[kW1]);
  ctx->ws.w1_inv = (float*)(p + offs[kW1Inv]);
  ctx->ws.w2 = (_Float16*)(p + offs[kW2]);
  ctx->ws.w2_inv = (float*)(p + offs[kW2Inv]);
  ctx->ws.q_norm = (float*)(p + offs[kGain]);
  ctx->ws.proj1_part = (float*)(p + offs[kPart1]);
  ctx->ws.ahat_hi = (_Float16*)(p + offs[kAHatHi]);
  ctx->ws.ahat_lo = (_Float16*)(p + offs[kAHatLo]);
  ctx->ws.ahat_inv = (float*)(p + offs[kAHatInv]);
  ctx->ws.rope_freq = (double*)(p + offs[kFreq]);
  ctx->ws.rope_cs = (float*)(p + offs[kCosSin]);
  ctx->ws.qpack = (void*)(p + offs[kQPack]);
  ctx->ws.qpack8 = (void*)(p + offs[kQPack8]);
  ctx->ws.w8 = (float*)(p + offs[kW8]);
  ctx->ws.row_tiles = (int64_t*)(p + offs[kRowTiles]);
  ctx->ws.wave_row = (int32_t*)(p + offs[kWaveRow]);
  ctx->ws.score_blocks = cus;
  ctx->ws.sub_keys = (uint32_t*)(p + offs[kSubKeys]);
  ctx->ws.sub_tiles = (uint2*)(p + offs[kSubTiles]);
  ctx->ws.res_count = (uint32_t*)(p + offs[kResCount]);
  ctx->ws.res_bits = (unsigned long long*)(p + offs[kResBits]);
  ctx->ws.tile_info = (uint2*)(p + offs[kTileInfo]);

  double freq[kRopeDim / 2];
  rope_frequencies(*cfg, freq);
  e = hipMemcpy(ctx->ws.rope_freq, freq, sizeof(freq), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = launch_pack_weights(*weights, ctx->ws, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(base);
    delete ctx;
    return hip_fail(e, "context initialisation");
  }
  *out = ctx;
  return FM_OK;
}

void fm_destroy(fm_ctx* ctx) {
  if (!ctx) return;
  if (ctx->ws_base) (void)hipFree(ctx->ws_base);
  delete ctx;
}

fm_status fm_prepare_query(fm_ctx* ctx, const float* hidden, const int64_t* positions, int32_t B, float* q_out,
                           float* w_out, void* stream) {
  clear_err();
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((st = check_shape(ctx, B, 0, false)) != FM_OK) return st;
  if (B == 0) return FM_OK;
  if (!hidden || !positions || !q_out || !w_out) return fail(FM_EINVAL, "null pointer to fm_prepare_query");
  if (!aligned(hidden, 16) || !aligned(q_out, 16) || !aligned(w_out, 16) || !aligned(positions, 8))
    return fail(FM_EINVAL, "hidden, q_out, w_out must be 16-byte aligned, positions 8-byte aligned");
  hipError_t e = fm::launch_prepare_query(ctx->cfg, ctx->weights, ctx->ws, ctx->max_batch, hidden, positions, B, q_out,
                                          w_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fm_prepare_query launch");
  return FM_OK;
}

static fm_status score_common(fm_ctx* ctx, const float* q, const float* w, const uint8_t* comp_k, int32_t B, int64_t N,
                              const int32_t* valid_n, fm_ensemble mode, float* scores, float* per_layer, void* stream,
                              bool fp8) {
  clear_err();
  const char* name = fp8 ? "fm_score_fp8" : "fm_score";
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((st = check_shape(ctx, B, N, true)) != FM_OK) return st;
  if (mode != FM_ENSEMBLE_MAX && mode != FM_ENSEMBLE_MEAN) return fail(FM_EINVAL, "unknown ensemble mode %d", (int)mode);
  if (B == 0 || N == 0) return FM_OK;
  if (!q || !w || !comp_k || !scores) return fail(FM_EINVAL, "null pointer to %s", name);
  if (!aligned(q, 16) || !aligned(w, 16) || !aligned(comp_k, 4) || !aligned(scores, 4) ||
      (per_layer && !aligned(per_layer, 4)) || (valid_n && !aligned(valid_n, 4)))
    return fail(FM_EINVAL, "q, w must be 16-byte aligned; comp_k, scores, per_layer, valid_n 4-byte aligned");
  hipError_t e = fp8 ? fm::launch_score_fp8(ctx->ws, q, w, comp_k, B, N, valid_n, (int)mode, scores, per_layer,
                                            (hipStream_t)stream)
                     : fm::launch_score(ctx->ws, q, w, comp_k, B, N, valid_n, (int)mode, scores, per_layer,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fp8 ? "fm_score_fp8 launch" : "fm_score launch");
  return FM_OK;
}

fm_status fm_score(fm_ctx* ctx, const float* q, const float* w, const uint8_t* comp_k, int32_t B, int64_t N,
                   const int32_t* valid_n, fm_ensemble mode, float* scores, float* per_layer, void* stream) {
  return score_common(ctx, q, w, comp_k, B, N, valid_n, mode, scores, per_layer, stream, false);
}

fm_status fm_score_fp8(fm_ctx* ctx, const float* q, const float* w, const uint8_t* comp_k, int32_t B, int64_t N,
                       const int32_t* valid_n, fm_ensemble mode, float* scores, float* per_layer, void* stream) {
  return score_common(ctx, q, w, comp_k, B, N, valid_n, mode, scores, per_layer, stream, true);
}

fm_status fm_score_threshold(fm_ctx* ctx, const float* q, const float* w, const uint8_t* comp_k, int32_t B, int64_t N,
                             const int32_t* valid_n, fm_ensemble mode, float threshold, float* scores, uint8_t* mask,
                             float* per_layer, void* stream) {
  clear_err();
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((st = check_shape(ctx, B, N, true)) != FM_OK) return st;
  if (mode != FM_ENSEMBLE_MAX && mode != FM_ENSEMBLE_MEAN) return fail(FM_EINVAL, "unknown ensemble mode %d", (int)mode);
  if (!std::isfinite(threshold)) return fail(FM_EINVAL, "threshold must be finite");
  if (B == 0 || N == 0) return FM_OK;
  if (!q || !w || !comp_k || !scores || !mask) return fail(FM_EINVAL, "null pointer to fm_score_threshold");
  if (!aligned(q, 16) || !aligned(w, 16) || !aligned(comp_k, 4) || !aligned(scores, 4) ||
      (per_layer && !aligned(per_layer, 4)) || (valid_n && !aligned(valid_n, 4)))
    return fail(FM_EINVAL, "q, w must be 16-byte aligned; comp_k, scores, per_layer, valid_n 4-byte aligned");
  hipError_t e = fm::launch_score_threshold(ctx->ws, q, w, comp_k, B, N, valid_n, (int)mode, threshold, scores, mask,
                                            per_layer, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fm_score_threshold launch");
  return FM_OK;
}

fm_status fm_set_score_events(fm_ctx* ctx, void* before, void* after) {
  clear_err();
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((before == nullptr) != (after == nullptr))
    return fail(FM_EINVAL, "fm_set_score_events takes two events or none");
  ctx->ws.score_ev[0] = (hipEvent_t)before;
  ctx->ws.score_ev[1] = (hipEvent_t)after;
  return FM_OK;
}

fm_status fm_select_topk(fm_ctx* ctx, const float* scores, int32_t B, int64_t N, const int32_t* valid_n,
                         int32_t top_k, uint8_t* mask, void* stream) {
  clear_err();
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((st = check_shape(ctx, B, N, true)) != FM_OK) return st;
  if (top_k < 0) return fail(FM_EINVAL, "top_k = %d < 0", top_k);
  if (B == 0 || N == 0) return FM_OK;
  if (!scores || !mask) return fail(FM_EINVAL, "null pointer to fm_select_topk");
  if (!aligned(scores, 4) || (valid_n && !aligned(valid_n, 4)))
    return fail(FM_EINVAL, "scores and valid_n must be 4-byte aligned");
  hipError_t e = fm::launch_select_topk(ctx->ws, scores, B, N, valid_n, top_k, mask, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fm_select_topk launch");
  return FM_OK;
}

fm_status fm_select_topk_static(const float* scores, int32_t B, int64_t N, const int32_t* valid_n, int32_t top_k,
                                uint8_t* mask, void* stream) {
  clear_err();
  if (B < 0 || B > 65535) return fail(FM_EINVAL, "B = %d outside [0, 65535]", B);
  if (N < 0 || N > (int64_t(1) << 26)) return fail(FM_EINVAL, "N = %lld outside [0, 2^26]", (long long)N);
  if (top_k < 0) return fail(FM_EINVAL, "top_k = %d < 0", top_k);
  const size_t need = sizeof(uint2) * (size_t)B * (size_t)fm::tile_info_stride(N);
  if (need > kStaticScratchBytes)
    return fail(FM_EINVAL, "B = %d, N = %lld need %zu scratch bytes; the static scratch holds %zu", B, (long long)N,
                need, kStaticScratchBytes);
  if (B == 0 || N == 0) return FM_OK;
  if (!scores || !mask) return fail(FM_EINVAL, "null pointer to fm_select_topk_static");
  if (!aligned(scores, 4) || (valid_n && !aligned(valid_n, 4)))
    return fail(FM_EINVAL, "scores and valid_n must be 4-byte aligned");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FM_EINVAL, "device %d beyond the %d supported", dev, kMaxDevices);
  void* p = nullptr;
  if ((e = static_scratch(dev, &p)) != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  fm::Workspace ws;
  ws.tile_info = (uint2*)p;
  e = fm::launch_select_topk(ws, scores, B, N, valid_n, top_k, mask, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fm_select_topk_static launch");
  return FM_OK;
}

fm_status fm_select_topk_subset(fm_ctx* ctx, const float* scores, int32_t B, int64_t N, const int32_t* subset,
                                const int32_t* n_subset, int32_t cap, int32_t top_k, int32_t* out, int32_t* n_out,
                                void* stream) {
  clear_err();
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((st = check_shape(ctx, B, N, true)) != FM_OK) return st;
  if (cap < 0 || top_k < 0) return fail(FM_EINVAL, "cap (%d) and top_k (%d) must be >= 0", cap, top_k);
  if (B == 0) return FM_OK;
  if (!n_out || (N > 0 && !scores) || (cap > 0 && !subset) || (top_k > 0 && !out))
    return fail(FM_EINVAL, "null pointer to fm_select_topk_subset");
  if (!aligned(scores, 4) || !aligned(subset, 4) || !aligned(n_subset, 4) || !aligned(out, 4) || !aligned(n_out, 4))
    return fail(FM_EINVAL, "scores, subset, n_subset, out, n_out must be 4-byte aligned");
  hipError_t e = fm::launch_select_topk_subset(ctx->ws, scores, B, N, subset, n_subset, cap, top_k, out, n_out,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fm_select_topk_subset launch");
  return FM_OK;
}

fm_status fm_select_threshold(fm_ctx* ctx, const float* scores, int32_t B, int64_t N, const int32_t* valid_n,
                              float threshold, uint8_t* mask, void* stream) {
  clear_err();
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((st = check_shape(ctx, B, N, true)) != FM_OK) return st;
  if (!std::isfinite(threshold)) return fail(FM_EINVAL, "threshold must be finite");
  if (B == 0 || N == 0) return FM_OK;
  if (!scores || !mask) return fail(FM_EINVAL, "null pointer to fm_select_threshold");
  if (!aligned(scores, 4) || (valid_n && !aligned(valid_n, 4)))
    return fail(FM_EINVAL, "scores and valid_n must be 4-byte aligned");
  hipError_t e = fm::launch_select_threshold(scores, B, N, valid_n, threshold, mask, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fm_select_threshold launch");
  return FM_OK;
}

fm_status fm_mask_logits(fm_ctx* ctx, void* logits, fm_dtype dtype, int32_t B, int32_t R, int64_t N,
                         const uint8_t* mask, void* stream) {
  clear_err();
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((st = check_shape(ctx, B, N, true)) != FM_OK) return st;
  if (dtype != FM_DTYPE_F32 && dtype != FM_DTYPE_BF16) return fail(FM_EINVAL, "unknown logit dtype %d", (int)dtype);
  if (R < 0) return fail(FM_EINVAL, "R (%d) must be >= 0", R);
  if (B == 0 || N == 0 || R == 0) return FM_OK;
  if (!logits || !mask) return fail(FM_EINVAL, "null pointer to fm_mask_logits");
  if (!aligned(logits, dtype == FM_DTYPE_F32 ? 4 : 2)) return fail(FM_EINVAL, "logits must be aligned to its element");
  hipError_t e = fm::launch_mask_logits(logits, (int)dtype, B, R, N, mask, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fm_mask_logits launch");
  return FM_OK;
}

fm_status fm_resident_delta(fm_ctx* ctx, const uint8_t* prev_mask, const uint8_t* mask, int32_t B, int64_t N,
                            int32_t cap, int32_t* resident, int32_t* n_resident, int32_t* entering,
                            int32_t* n_entering, int32_t* leaving, int32_t* n_leaving, void* stream) {
  clear_err();
  fm_status st = check_ctx(ctx);
  if (st != FM_OK) return st;
  if ((st = check_shape(ctx, B, N, true)) != FM_OK) return st;
  if (cap < 0) return fail(FM_EINVAL, "cap = %d must be >= 0", cap);
  if ((entering == nullptr) != (n_entering == nullptr) || (leaving == nullptr) != (n_leaving == nullptr))
    return fail(FM_EINVAL, "each optional list comes with its count array (both or neither)");
  if (B == 0 || N == 0) return FM_OK;
  if (!mask || !resident || !n_resident) return fail(FM_EINVAL, "null pointer to fm_resident_delta");
  if (!aligned(resident, 4) || !aligned(n_resident, 4) || (entering && (!aligned(entering, 4) || !aligned(n_entering, 4))) ||
      (leaving && (!aligned(leaving, 4) || !aligned(n_leaving, 4))))
    return fail(FM_EINVAL, "index lists and counts must be 4-byte aligned");
  hipError_t e = fm::launch_resident_delta(ctx->ws, prev_mask, mask, B, N, cap, resident, n_resident, entering,
                                           n_entering, leaving, n_leaving, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fm_resident_delta launch");
  return FM_OK;
}

}  // extern "C"
