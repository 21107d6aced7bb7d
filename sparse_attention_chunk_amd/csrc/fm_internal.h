// Internal declarations of libfm: compiled dimensions, the context layout and
// the launchers each kernel file provides to the C ABI layer (fm_api.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "fm.h"
#include "fm_index.h"

namespace fm {

// Compiled layer dimensions (README "Architecture"; HEAD_DIM from the
// 132-byte record of "compressed_k format").
constexpr int kLayers = 3;
constexpr int kHidden = 4096;
constexpr int kQLora = 1024;
constexpr int kHeads = 64;
constexpr int kHeadDim = 128;
constexpr int kRopeDim = 64;
constexpr int kRecord = kHeadDim + 4;

// First projection: wq_a rows [0, 1024) and weights_proj rows [1024, 1088)
// share one pass over `hidden`.  A wave covers 16 outputs x up to 32 batch
// rows over one 512-wide K slice (more rows go to further wave groups); the
// slice partial sums are added in slice order by the next kernel, so the
// weights stream from HBM once.
constexpr int kProj1Out = kQLora + kHeads;
constexpr int kProjRowsPerWave = 32;
constexpr int kSliceK = 512;
constexpr int kSliceChunks = kSliceK / 128;

inline int proj_row_groups(int B) { return (B + kProjRowsPerWave - 1) / kProjRowsPerWave; }
// K slices of the first projection (K = 4096).
inline int proj1_splits(int) { return kHidden / kSliceK; }

// Score kernel: per request row the packed fp16 queries are 48 MFMA
// fragments (3 layers x 4 head tiles x 4 k-steps) of 64 lanes x 8 halves,
// then one fp8 fragment (64 lanes x 32 bytes) of the per-layer weighted
// query sums in three e4m3 parts and their three power-of-two scales; a
// row takes kQFrags 1 KB units (the last holds the fp8 fragment's block-scale
// codes).
constexpr int kQHeadFrags = kLayers * 4 * 4;
constexpr int kQFrags = kQHeadFrags + 3;
// fp8 score path: per request row 24 fragments of 64 lanes x 32 e4m3 bytes
// (3 layers x 4 head tiles x {hi, lo} parts), then one fragment of the
// per-layer weighted query sums in three parts; per row (kW8Row floats) the
// halved head weights of each layer with each head's query scale folded in,
// then the linear fragment's 64 per-lane block-scale codes (int32).
constexpr int kQ8HeadFrags = kLayers * 4 * 2;
constexpr int kQ8Frags = kQ8HeadFrags + 1;
constexpr int kW8Row = kLayers * kHeads + 64;
// The score kernel runs one block of 4 waves per compute unit; each wave
// takes an equal share of the row-major list of 16-chunk tiles.
constexpr int kMaxScoreBlocks = 1024;

// Histogram bins of the exact selections.
constexpr int kSelBins = 2048;

// Subset top-K: lists of up to kSubFastCap entries take the scan + finish
// path, with their keys and tile words in workspace buffers; longer lists
// are selected by one block per row that gathers the keys in every pass.
constexpr int kSubFastCap = 32768;

// Resident-set compaction: a block covers kResSlice chunks of one row.
constexpr int kResSlice = 4096;

// Top-K selection: the scan kernel writes a 64-bit word per tile of 16 or
// more chunks (histogram bins and positions of its largest scores), in rows
// of tile_info_stride(N) words (fm_index.h).
using idx::tile_info_stride;

struct Workspace {
  // Weights packed at context creation: each row scaled by a power of two
  // and split into f16 hi + lo parts, in 16-row tiles of 2 KB k-steps (the
  // projection kernel's operand order), with each row's 2^-e.
  _Float16* w1 = nullptr;        // [3][kProj1Out * kHidden * 2]: wq_a rows, then weights_proj rows
  float* w1_inv = nullptr;       // [3][kProj1Out]
  _Float16* w2 = nullptr;        // [3][kHeads * kHeadDim * kQLora * 2]: wq_b
  float* w2_inv = nullptr;       // [3][kHeads * kHeadDim]
  float* q_norm = nullptr;       // [3][kQLora] RMSNorm gains
  float* proj1_part = nullptr;   // [proj1_splits(B)][3][B][kProj1Out]
  _Float16* ahat_hi = nullptr;   // [3][max_batch][kQLora]: RMSNorm output, each 128-chunk of a row scaled by a
  _Float16* ahat_lo = nullptr;   //   power of two and split into f16 hi + lo parts (wq_b's operand)
  float* ahat_inv = nullptr;     // [3][max_batch][kQLora / 128]: 2^-e of each chunk
  double* rope_freq = nullptr;   // [kRopeDim / 2]
  float* rope_cs = nullptr;      // [max_batch][kRopeDim / 2][2]: cos, sin of position * freq
  void* qpack = nullptr;         // [max_batch][kQFrags][64][8] fp16
  void* qpack8 = nullptr;        // [max_batch][kQ8Frags][64][32] e4m3
  float* w8 = nullptr;           // [max_batch][kW8Row]
  int64_t* row_tiles = nullptr;  // [max_batch + 1]: first tile of each row in the list of valid tiles
  int32_t* wave_row = nullptr;   // [4 * score_blocks]: row holding each wave's first tile
  int score_blocks = 0;          // compute units of the device
  uint32_t* sub_keys = nullptr;  // [max_batch][kSubFastCap]: keys of the list positions (scan + finish path)
  uint2* sub_tiles = nullptr;    // [max_batch][kSubFastCap / 16]: their tile words
  uint32_t* res_count = nullptr; // [max_batch][ceil(max_n / kResSlice)][3]: set sizes per slice
  unsigned long long* res_bits = nullptr;  // [max_batch][ceil(max_n / kResSlice) * 256]: per 16 chunks, the
                                           //   three sets' bits (16 each), from the count pass
  uint2* tile_info = nullptr;    // [max_batch][tile_info_stride(max_n)]: per tile, for the top-K finish
  // Caller's timing events (fm_set_score_events), recorded on the call's
  // stream right before and right after the score kernel's own launch; null
  // when unset.
  hipEvent_t score_ev[2] = {nullptr, nullptr};
};

// Records the workspace's score events around one launch (when set).
inline void record_score_event(const Workspace& ws, int which, hipStream_t stream) {
  if (ws.score_ev[which]) (void)hipEventRecord(ws.score_ev[which], stream);
}

// Launchers.  Shapes are validated by the caller; each returns the launch
// status (hipGetLastError after the launches).

// Packs the caller's fp32 weights into the workspace (hi/lo parts, row
// scales, gains).
hipError_t launch_pack_weights(const fm_weights& wts, const Workspace& ws, hipStream_t stream);
hipError_t launch_prepare_query(const fm_config& cfg, const fm_weights& wts, const Workspace& ws, int max_batch,
                                const float* hidden, const int64_t* positions, int B, float* q_out, float* w_out,
                                hipStream_t stream);

hipError_t launch_score(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B, int64_t N,
                        const int32_t* valid_n, int mode, float* scores, float* per_layer, hipStream_t stream);
hipError_t launch_score_fp8(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B,
                            int64_t N, const int32_t* valid_n, int mode, float* scores, float* per_layer,
                            hipStream_t stream);
// Shared by both score launchers: with valid_n, plans the ragged tile list
// (row_tiles, wave_row) and writes -inf past each row's valid_n; returns the
// tile list to walk (row_tiles, or null and total_tiles for full rows).
hipError_t launch_score_plan(const Workspace& ws, const int32_t* valid_n, int B, int64_t N, float* scores,
                             float* per_layer, hipStream_t stream, const int64_t** row_tiles, int64_t* total_tiles);

hipError_t launch_select_topk(const Workspace& ws, const float* scores, int B, int64_t N, const int32_t* valid_n,
                              int32_t top_k, uint8_t* mask, hipStream_t stream);

// The score pass writing the threshold keep mask as well (scores as
// launch_score; mask[b][n] = score > threshold, 0 at or beyond valid_n).
hipError_t launch_score_threshold(const Workspace& ws, const float* q, const float* w, const uint8_t* comp_k, int B,
                                  int64_t N, const int32_t* valid_n, int mode, float threshold, float* scores,
                                  uint8_t* mask, float* per_layer, hipStream_t stream);

// Subset top-K: the scan + finish path (cap <= kSubFastCap) and the entry
// that picks it or the long-list path.
hipError_t launch_select_topk_subset_fast(const Workspace& ws, const float* scores, int B, int64_t N,
                                          const int32_t* subset, const int32_t* n_subset, int32_t cap, int32_t top_k,
                                          int32_t* out, int32_t* n_out, hipStream_t stream);
hipError_t launch_select_topk_subset(const Workspace& ws, const float* scores, int B, int64_t N,
                                     const int32_t* subset, const int32_t* n_subset, int32_t cap, int32_t top_k,
                                     int32_t* out, int32_t* n_out, hipStream_t stream);

hipError_t launch_select_threshold(const float* scores, int B, int64_t N, const int32_t* valid_n, float threshold,
                                   uint8_t* mask, hipStream_t stream);

hipError_t launch_mask_logits(void* logits, int dtype, int B, int R, int64_t N, const uint8_t* mask,
                              hipStream_t stream);

hipError_t launch_resident_delta(const Workspace& ws, const uint8_t* prev, const uint8_t* mask, int B, int64_t N,
                                 int32_t cap, int32_t* resident, int32_t* n_resident, int32_t* entering,
                                 int32_t* n_entering, int32_t* leaving, int32_t* n_leaving, hipStream_t stream);

}  // namespace fm

struct fm_ctx {
  int device = 0;
  fm_config cfg{};
  fm_weights weights{};
  int32_t max_batch = 0;
  int64_t max_n = 0;
  fm::Workspace ws{};
  void* ws_base = nullptr;  // one allocation holding every workspace buffer
  size_t ws_bytes = 0;
};
