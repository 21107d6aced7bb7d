// Per-step top-K confined to a subset of the chunks (FlashMemory-DeepSeek-V4
// model card, "How it works": the Lightning Indexer's top-512 of every decode
// step runs only over the resident_set that the Memory Indexer recalled).
//
// Per row: the subset is a list of chunk indices (the resident set, as
// fm_resident_delta writes it); the step's scores cover all N chunks.  The
// result is the top_k subset entries by score, ties going to the earlier
// list position (the lower chunk index when the list is ascending), written
// as chunk indices in list order.  Entries outside [0, N) are never chosen.
//
// Lists of up to kSubFastCap (32768) entries take the row top-K's tile scan
// and finish (fm_select.hip).  This file holds the path for longer lists: one
// block of 1024 threads per row; position p of the list is handled by thread
// p mod 1024 (coalesced list reads), in rounds of 1024 positions, its key
// (the order-preserving uint32 of its score) gathered again in every pass,
// eight rounds of loads at a time.  An exact radix selection over the whole
// list gives the k-th largest key T and the last position kept among the
// keys equal to T, and the chosen entries are written in list order: per
// round each wave ballots its 64 positions, the counts of all (round, wave)
// pairs are scanned once, each chosen position is written at its wave's
// offset plus the chosen lanes below it, and a last pass replaces every
// written position by its chunk index.
#include "fm_radix.h"

namespace fm {
namespace {

using namespace radix;

constexpr int kSubThreads = 1024;
constexpr int kSubWaves = kSubThreads / 64;
constexpr int kSubGroupRounds = 64;  // rounds of 1024 positions per compaction group

// Exclusive block scan of one count per thread; also the block total.  Ends
// after a barrier that follows every read of s_w.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_w, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_prefix_sum(v);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  uint32_t below = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSubWaves; ++w) {
    const uint32_t x = s_w[w];
    below += w < wave ? x : 0u;
    all += x;
  }
  __syncthreads();
  *total = all;
  return below + incl - v;
}

constexpr int kSubBatch = 8;  // rounds of loads in flight per pass

__device__ __forceinline__ bool in_range(int32_t i, int64_t N) { return i >= 0 && (int64_t)i < N; }

// grid = B, block = 1024: the selection of row b's list (cap > kSubFastCap).
__global__ __launch_bounds__(kSubThreads) void sel_subset_kernel(const float* __restrict__ scores, int64_t N,
                                                                 const int32_t* __restrict__ subset,
                                                                 const int32_t* __restrict__ n_subset, int32_t cap,
                                                                 int32_t top_k, int32_t* __restrict__ out,
                                                                 int32_t* __restrict__ n_out) {
  __shared__ __attribute__((aligned(16))) uint32_t h[2 * kSelBins];
  __shared__ uint32_t s_wtot[kSubWaves];
  __shared__ uint32_t s_out[3];
  __shared__ uint32_t s_cnt[kSubGroupRounds * kSubWaves];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t n64 = n_subset ? (int64_t)n_subset[b] : (int64_t)cap;
  const uint32_t n = (uint32_t)(n64 < 0 ? 0 : (n64 > cap ? cap : n64));  // below 2^31
  const uint32_t rounds = (n + kSubThreads - 1) / kSubThreads;
  const int32_t* srow = subset + (size_t)b * cap;
  const float* row = scores + (size_t)b * N;

  uint32_t nvalid = 0;
  for (uint32_t p = t; p < n; p += kSubThreads) nvalid += in_range(srow[p], N) ? 1u : 0u;
  // fn(key, position) for each of this thread's valid entries.
  auto each_entry = [&](auto fn) {
    for (uint32_t j0 = 0; j0 < rounds; j0 += kSubBatch) {
      int32_t bi[kSubBatch];
      float bv[kSubBatch];
#pragma unroll
      for (int u = 0; u < kSubBatch; ++u) {
        const uint32_t p = (j0 + u) * kSubThreads + t;
        bi[u] = p < n ? srow[p] : -1;
      }
#pragma unroll
      for (int u = 0; u < kSubBatch; ++u) bv[u] = in_range(bi[u], N) ? row[bi[u]] : 0.f;
#pragma unroll
      for (int u = 0; u < kSubBatch; ++u)
        if (in_range(bi[u], N)) fn(order_key(bv[u]), (j0 + u) * kSubThreads + t);
    }
  };
  auto each = [&](auto f) { each_entry([&](uint32_t k, uint32_t p) { f(make_uint2(k, p)); }); };

  uint32_t V;
  (void)block_exclusive_scan(nvalid, s_wtot, &V);
  const uint32_t k = (uint32_t)top_k < V ? (uint32_t)top_k : V;
  if (t == 0) n_out[b] = (int32_t)k;
  if (k == 0) return;
  int32_t* orow = out + (size_t)b * top_k;
  const uint64_t below_me = (1ull << lane) - 1ull;
  uint32_t T = 0, last = 0xffffffffu;  // k == V: every valid entry is chosen
  if (k < V) radix_select<kSubThreads>(each, k, index_bits((int64_t)n), h, s_wtot, s_out, &T, &last);
  auto chosen = [&](uint32_t key, uint32_t p) { return key > T || (key == T && p <= last); };

  // Chosen positions in list order, in groups of kSubGroupRounds rounds:
  // out[slot] = position first, the chunk index after.
  uint32_t base = 0;
  for (uint32_t g0 = 0; g0 < rounds; g0 += kSubGroupRounds) {
    const uint32_t gr = rounds - g0 < (uint32_t)kSubGroupRounds ? rounds - g0 : (uint32_t)kSubGroupRounds;
    uint64_t mine = 0;  // bit j: this thread's entry of round g0 + j is chosen
    each_entry([&](uint32_t key, uint32_t p) {
      const uint32_t j = p / kSubThreads - g0;
      if (j < gr && chosen(key, p)) mine |= 1ull << j;
    });
    for (uint32_t j = 0; j < gr; ++j) {
      const uint64_t m = __ballot((mine >> j) & 1ull);
      if (lane == 0) s_cnt[j * kSubWaves + wave] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    const uint32_t c = (uint32_t)t < gr * kSubWaves ? s_cnt[t] : 0u;
    uint32_t tot;
    const uint32_t off = block_exclusive_scan(c, s_wtot, &tot);
    if ((uint32_t)t < gr * kSubWaves) s_cnt[t] = off;
    __syncthreads();
    for (uint32_t j = 0; j < gr; ++j) {
      const bool cj = (mine >> j) & 1ull;
      const uint64_t m = __ballot(cj);
      if (cj) orow[base + s_cnt[j * kSubWaves + wave] + (uint32_t)__popcll(m & below_me)] =
          (int32_t)((g0 + j) * kSubThreads + t);
    }
    base += tot;
    __syncthreads();  // s_cnt is rewritten by the next group; the positions are visible to the block
  }
  for (uint32_t s_ = t; s_ < k; s_ += kSubThreads) orow[s_] = srow[orow[s_]];
}

}  // namespace

hipError_t launch_select_topk_subset(const Workspace& ws, const float* scores, int B, int64_t N,
                                     const int32_t* subset, const int32_t* n_subset, int32_t cap, int32_t top_k,
                                     int32_t* out, int32_t* n_out, hipStream_t stream) {
  if (cap <= kSubFastCap) return launch_select_topk_subset_fast(ws, scores, B, N, subset, n_subset, cap, top_k, out,
                                                                 n_out, stream);
  hipLaunchKernelGGL(sel_subset_kernel, dim3(B), dim3(kSubThreads), 0, stream, scores, N, subset, n_subset, cap,
                     top_k, out, n_out);
  return hipGetLastError();
}

}  // namespace fm
