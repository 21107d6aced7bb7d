/*
 * fm.h - C ABI of the FlashMemory Memory-Indexer scoring pass for MI355X
 * (gfx950).
 *
 * The pass is defined by the FlashMemory-DeepSeek-V4 README ("FlashMemory
 * DS-V4 Retriever"):
 *   - "Usage": inputs hidden [B, 4096] (decode-token hidden state),
 *     comp_k [B, N, 132] uint8 (compressed CSA keys), positions [B] int64;
 *     outputs per-layer sigmoid scores {l10, l12, l20} [B, N], an ensemble
 *     [B, N] (mode max or mean) and a boolean keep mask from top_k=... or
 *     threshold=...;
 *   - "compressed_k format": one chunk = HEAD_DIM + 4 = 132 bytes, 128
 *     float8_e4m3 codes followed by a float32 scale;
 *   - "Architecture": the query branch (wq_a, RMSNorm, wq_b, reshape,
 *     YaRN RoPE on the last 64 dims, normalized Walsh-Hadamard), the weight
 *     branch (weights_proj times HEAD_DIM^-0.5 N_HEADS^-0.5) and
 *     score = sigmoid(sum_heads relu(k . q_h) * w_h);
 *   - "Joint checkpoint + ensemble": three independent layers (l10, l12,
 *     l20), combined per chunk by max (default) or mean;
 *   - "Inference flow": keep mask = top-K of the scores, or score > thresh.
 *
 * Conventions shared by every call:
 *   - Pointers named as device pointers must be device memory of the GPU
 *     that was current when the context was created; host pointers are
 *     named as such.  The caller owns every buffer.  fm_create copies the
 *     weights into the context (in its own packed form): the weight buffers
 *     are not used after fm_create returns.
 *   - Row-major layouts, no padding: [B, N] has row stride N.
 *   - Float buffers must be 4-byte aligned, positions 8-byte aligned,
 *     comp_k 4-byte aligned (its records sit at a 132-byte stride).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising.  Inputs must stay valid
 *     until that work completes.  One context serves one stream at a time
 *     (its workspace is shared by the calls).
 *   - No call allocates device memory after fm_create.
 *   - Errors: every argument is checked before anything is enqueued; a
 *     failing call enqueues nothing and returns a negative fm_status, with
 *     a message in fm_last_error().  FM_EHIP means a HIP runtime call or a
 *     launch failed (message from hipGetErrorString).
 *   - B == 0 or N == 0 is an empty problem: FM_OK, nothing enqueued.
 */
#ifndef FM_H_
#define FM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fm_ctx fm_ctx; /* opaque */

typedef enum {
  FM_OK = 0,
  FM_EINVAL = -1,        /* bad argument: null pointer, out-of-range size, misalignment */
  FM_EUNSUPPORTED = -2,  /* dimensions other than the compiled ones */
  FM_ENOMEM = -3,        /* workspace allocation failed in fm_create */
  FM_EHIP = -4           /* HIP runtime or launch failure */
} fm_status;

/* Cross-layer ensemble ("Joint checkpoint + ensemble"): max is the union
 * and the default; mean is the arithmetic mean of the three sigmoid scores. */
typedef enum { FM_ENSEMBLE_MAX = 0, FM_ENSEMBLE_MEAN = 1 } fm_ensemble;

/* Element type of attention logits (fm_mask_logits). */
typedef enum { FM_DTYPE_F32 = 0, FM_DTYPE_BF16 = 1 } fm_dtype;

/* Layer dimensions and constants ("Architecture").  The compiled kernels
 * support exactly n_layers 3, hidden 4096, q_lora_rank 1024, n_heads 64,
 * head_dim 128, rope_dim 64; other values give FM_EUNSUPPORTED.
 * yarn_factor 1 is plain RoPE with frequencies base^(-2j/rope_dim); above 1
 * the frequencies blend linearly in j from base^(-2j/rope_dim) (below the
 * fast correction bound, from beta_fast) to that divided by yarn_factor
 * (above the slow bound, from beta_slow), both bounds taken over
 * yarn_orig_ctx. */
typedef struct {
  int32_t n_layers;      /* 3 */
  int32_t hidden;        /* 4096 */
  int32_t q_lora_rank;   /* 1024 */
  int32_t n_heads;       /* 64 */
  int32_t head_dim;      /* 128 */
  int32_t rope_dim;      /* 64: RoPE turns the last rope_dim dims of each head */
  float rms_eps;         /* 1e-6 */
  double rope_base;      /* 160000 */
  double yarn_factor;    /* 1 = plain RoPE */
  int64_t yarn_orig_ctx; /* 65536 */
  double yarn_beta_fast; /* 32 */
  double yarn_beta_slow; /* 1 */
} fm_config;

/* Device fp32 weights of the three layers, in the order l10, l12, l20,
 * each row-major [out][in] (a linear map in -> out, no bias):
 *   wq_a   [q_lora_rank][hidden]
 *   q_norm [q_lora_rank]                 RMSNorm gain
 *   wq_b   [n_heads * head_dim][q_lora_rank]; output row 128*h + d is
 *          element d of head h
 *   w_proj [n_heads][hidden]             weights_proj */
typedef struct {
  const float* wq_a[3];
  const float* q_norm[3];
  const float* wq_b[3];
  const float* w_proj[3];
} fm_weights;

/* Fills *cfg with the defaults listed in fm_config. */
void fm_config_default(fm_config* cfg);

/* Creates a context on the current HIP device.  Checks cfg, derives the
 * RoPE/YaRN frequencies (in double precision), allocates the workspace for
 * up to max_batch rows of up to max_n chunks and packs the weights into it:
 * every weight row is scaled by a power of two and split into two f16
 * parts (hi + lo, 4 bytes per weight), so that the projections run on the
 * f16 MFMA at about fp32 accuracy.  Synchronises the device before
 * returning.  max_batch in [1, 4096], max_n in [1, 2^26].  On success *out
 * receives the context. */
fm_status fm_create(const fm_config* cfg, const fm_weights* weights, int32_t max_batch, int64_t max_n,
                    fm_ctx** out);

/* Frees the workspace.  Waits for nothing: the caller synchronises any
 * stream still using the context first.  NULL is a no-op. */
void fm_destroy(fm_ctx* ctx);

/* Query and weight branches ("Architecture"), all three layers.
 *   hidden    device fp32 [B][hidden]
 *   positions device int64 [B], token position of each row (>= 0)
 *   q_out     device fp32 [3][B][n_heads][head_dim]: q after RoPE and the
 *             normalized Hadamard transform
 *   w_out     device fp32 [3][B][n_heads]: fused_w
 * B in [0, max_batch]. */
fm_status fm_prepare_query(fm_ctx* ctx, const float* hidden, const int64_t* positions, int32_t B, float* q_out,
                           float* w_out, void* stream);

/* Per-layer score and ensemble ("Architecture" score line, "Joint checkpoint
 * + ensemble").
 *   q, w      device fp32, as written by fm_prepare_query; q is rounded once
 *             to f16 for the MFMA, so its entries must stay within the f16
 *             range (|q| <= 65504), and that rounding moves each logit by
 *             about 2^-11 of its size: the score tolerance holds for q of the
 *             prepared queries' size (order one, a normalised transform of
 *             RMS-normalised projections)
 *   comp_k    device uint8 [B][N][132] ("compressed_k format"): bytes 0..127
 *             are OCP float8 e4m3fn codes, bytes 128..131 a little-endian
 *             fp32 scale; k = decode(code) * scale
 *   valid_n   device int32 [B] or NULL (= N for every row): chunks at index
 *             >= valid_n[b] are not read; values are clamped to [0, N]
 *   mode      FM_ENSEMBLE_MAX or FM_ENSEMBLE_MEAN
 *   scores    device fp32 [B][N]: ensemble score in [0, 1]; -inf at or
 *             beyond valid_n
 *   per_layer device fp32 [3][B][N] or NULL: each layer's sigmoid score
 *             (the pages' {"l10","l12","l20"} dict); -inf beyond valid_n
 * B in [0, max_batch], N in [0, max_n]. */
fm_status fm_score(fm_ctx* ctx, const float* q, const float* w, const uint8_t* comp_k, int32_t B, int64_t N,
                   const int32_t* valid_n, fm_ensemble mode, float* scores, float* per_layer, void* stream);

/* fm_score with the threshold keep mask ("Usage" select_topk with
 * threshold=...; "Inference flow" sigmoid > thresh) written by the score
 * pass itself: mask[b][n] = score > threshold (strict), 0 at or beyond
 * valid_n.  Arguments as fm_score plus threshold (finite) and mask (device
 * uint8 [B][N]).  The result equals fm_score followed by
 * fm_select_threshold. */
fm_status fm_score_threshold(fm_ctx* ctx, const float* q, const float* w, const uint8_t* comp_k, int32_t B, int64_t N,
                             const int32_t* valid_n, fm_ensemble mode, float threshold, float* scores, uint8_t* mask,
                             float* per_layer, void* stream);

/* fm_score on the fp8 matrix cores: the native-FP8 indexer form that the
 * FlashMemory DS-V4 Retriever README's "Is / is not" section names for
 * production.  Same arguments, outputs and error behaviour as fm_score.
 * The stored e4m3
 * codes enter the fp8 MFMA directly; each head's query is scaled by a power
 * of two and split into two e4m3 parts (hi + lo, about 8 significant bits;
 * relative error at most 2^-8 per element), so the scores are less precise
 * than fm_score's (measured within 6e-4 of the fp64 result on the synthetic
 * workloads, against 2.3e-4) and stay within the same 2e-3 bound. */
fm_status fm_score_fp8(fm_ctx* ctx, const float* q, const float* w, const uint8_t* comp_k, int32_t B, int64_t N,
                       const int32_t* valid_n, fm_ensemble mode, float* scores, float* per_layer, void* stream);

/* Keep mask of the top_k highest scores of each row ("Usage" top_k=...;
 * "Inference flow" top-K).  Ties are broken towards the lower chunk index,
 * so the mask is unique; top_k >= valid_n keeps every valid chunk; top_k 0
 * keeps none; chunks at or beyond valid_n are never kept.
 *   scores  device fp32 [B][N] (finite or -inf; NaN is not ordered)
 *   valid_n device int32 [B] or NULL, as in fm_score
 *   mask    device uint8 [B][N], written 1 (keep) or 0
 * top_k >= 0. */
fm_status fm_select_topk(fm_ctx* ctx, const float* scores, int32_t B, int64_t N, const int32_t* valid_n,
                         int32_t top_k, uint8_t* mask, void* stream);

/* fm_select_topk without a context and without any allocation, for callers
 * that cannot allocate (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus ctx), result
 * and tie-breaking as fm_select_topk; its scratch (the scan's tile words,
 * 8 bytes per 16 chunks of each row) is a static 8 MiB device array that
 * each GPU holds until the process ends: B * 8 * (ceil(N / 16) rounded up
 * to even) must not exceed 8 MiB (B = 30, N = 262144 needs 3.75 MiB), else
 * FM_EINVAL.  B in [0, 65535], N in [0, 2^26].  Every call on a GPU shares
 * that GPU's scratch: calls that overlap on one GPU (other streams, other
 * threads) race; the first call on a device looks the array's address up.
 * Rows of at most 8192 chunks are selected in one launch that uses no
 * scratch (the size limit still applies). */
fm_status fm_select_topk_static(const float* scores, int32_t B, int64_t N, const int32_t* valid_n, int32_t top_k,
                                uint8_t* mask, void* stream);

/* Per-step top-K confined to a subset of the chunks (model card "How it
 * works", Level 2: the Lightning Indexer's top-512 runs only over the
 * resident_set that the Memory Indexer recalled).  The pages define the
 * selection, not the step's score function: the scores are an input.
 *   scores    device fp32 [B][N], the step's score of every chunk (finite or
 *             -inf; NaN is not ordered)
 *   subset    device int32 [B][cap]: row b's chunk indices (its resident
 *             set, e.g. fm_resident_delta's list), distinct; entries outside
 *             [0, N) are never chosen.  May be NULL when cap is 0
 *   n_subset  device int32 [B] or NULL (= cap): entries used per row,
 *             clamped to [0, cap]
 *   top_k     entries to choose per row (>= 0)
 *   out       device int32 [B][top_k]: the chosen chunk indices in subset
 *             order (ascending when the subset is); entries past n_out[b]
 *             are not written
 *   n_out     device int32 [B]: min(top_k, valid entries of row b)
 * The chosen entries are the top_k by score; ties go to the earlier subset
 * position (the lower chunk index for an ascending subset), so the result
 * is unique.  B in [0, max_batch], N in [0, max_n], cap >= 0. */
fm_status fm_select_topk_subset(fm_ctx* ctx, const float* scores, int32_t B, int64_t N, const int32_t* subset,
                                const int32_t* n_subset, int32_t cap, int32_t top_k, int32_t* out, int32_t* n_out,
                                void* stream);

/* Keep mask score > threshold, strictly ("Usage" threshold=...;
 * "Inference flow" sigmoid > thresh).  Chunks at or beyond valid_n are
 * never kept.  threshold must be finite. */
fm_status fm_select_threshold(fm_ctx* ctx, const float* scores, int32_t B, int64_t N, const int32_t* valid_n,
                              float threshold, uint8_t* mask, void* stream);

/* Resident set and recall delta of a retrieval cycle (model card "How it
 * works": the Memory Indexer's selection is the resident_set recalled from
 * CPU to GPU every 64 decode steps; README "Inference flow": a cycle's keep
 * mask holds for the next 64 steps).  Per row, in ascending chunk index:
 *   resident = chunks set in mask
 *   entering = chunks set in mask and not in prev_mask   (to recall)
 *   leaving  = chunks set in prev_mask and not in mask   (to evict)
 * A mask byte is set when it is non-zero.
 *   prev_mask   device uint8 [B][N], the previous cycle's mask, or NULL
 *               (first cycle: entering = resident, leaving empty)
 *   mask        device uint8 [B][N], this cycle's mask
 *   cap         capacity of each list per row (>= 0)
 *   resident    device int32 [B][cap]; n_resident device int32 [B]
 *   entering    device int32 [B][cap] or NULL; n_entering [B] (NULL with it)
 *   leaving     device int32 [B][cap] or NULL; n_leaving [B] (NULL with it)
 * The counts are the sets' full sizes; a list longer than cap holds its
 * first cap indices.  B in [0, max_batch], N in [0, max_n]. */
fm_status fm_resident_delta(fm_ctx* ctx, const uint8_t* prev_mask, const uint8_t* mask, int32_t B, int64_t N,
                            int32_t cap, int32_t* resident, int32_t* n_resident, int32_t* entering,
                            int32_t* n_entering, int32_t* leaving, int32_t* n_leaving, void* stream);

/* Attention-logit masking over a retrieval cycle (README "Inference flow":
 * for the next 64 decode steps the attention logits of unselected chunks
 * are -inf; "What this simulates": a masked chunk contributes nothing to
 * attention, as if its KV were not loaded).  In place:
 *   logits  device [B][R][N] of dtype (fp32 or bf16): R logit rows per
 *           request row (heads, query positions); set to -inf where
 *           mask[b][n] == 0, untouched where it is non-zero
 *   mask    device uint8 [B][N], e.g. fm_select_topk's keep mask
 * B in [0, max_batch], N in [0, max_n], R >= 0; logits aligned to its
 * element size. */
fm_status fm_mask_logits(fm_ctx* ctx, void* logits, fm_dtype dtype, int32_t B, int32_t R, int64_t N,
                         const uint8_t* mask, void* stream);

/* Timing hook for the score kernel alone (not a step of the pass: for
 * measuring the dominant kernel against its roofline).  With two events
 * set, every later fm_score, fm_score_threshold and fm_score_fp8 on ctx
 * records `before` on its stream right before the score kernel's launch
 * (after the query packing and the ragged-row planning) and `after` right
 * after it, so hipEventElapsedTime(before, after) is that launch's
 * duration.
 *   before, after  hipEvent_t of the context's device, created and owned
 *                  by the caller, valid while set; both NULL clears them
 * A score call that enqueues nothing (B == 0 or N == 0, or an argument
 * error) records nothing, so the events keep their last timestamps.  One
 * NULL and one not gives FM_EINVAL.  A failing record makes the score call
 * return FM_EHIP (after its launches were enqueued). */
fm_status fm_set_score_events(fm_ctx* ctx, void* before, void* after);

/* Message of the last failing call on this thread ("" if none); valid until
 * the next fm_* call on this thread. */
const char* fm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FM_H_ */
