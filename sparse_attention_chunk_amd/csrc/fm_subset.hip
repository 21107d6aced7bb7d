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
// One block of 1024 threads per row; position p of the list is handled by
// thread p mod 1024 (coalesced list reads).  The keys (order-preserving
// uint32 of the gathered scores) and a validity bitmap are kept in LDS when
// the list fits, else every pass gathers them again.  An exact radix
// selection gives the k-th largest key T and the last position kept among
// the keys equal to T.  The chosen entries are then written in list order:
// per round of 1024 positions each wave ballots its 64, the counts of all
// (round, wave) pairs are scanned once, and each entry lands at its wave's
// offset plus the chosen lanes below it.
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

// LDS: keys and validity in dynamic LDS (4 cap bytes of keys, then the
// bitmap, 128 bytes per round of 1024 positions, as the launch sizes it).
template <bool LDS>
__global__ __launch_bounds__(kSubThreads) void sel_subset_kernel(const float* __restrict__ scores, int64_t N,
                                                                 const int32_t* __restrict__ subset,
                                                                 const int32_t* __restrict__ n_subset, int32_t cap,
                                                                 int32_t top_k, int32_t* __restrict__ out,
                                                                 int32_t* __restrict__ n_out) {
  extern __shared__ uint32_t s_keys[];
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
  uint32_t* s_valid = s_keys + (LDS ? (size_t)cap : 0);  // bit p % 32 of word p / 32

  // The chunk index at position p, when it is in [0, N), and its key.
  auto gather = [&](uint32_t p, uint32_t& key) -> bool {
    const int32_t i = srow[p];
    if (i < 0 || (int64_t)i >= N) return false;
    key = order_key(row[i]);
    return true;
  };
  uint32_t nvalid = 0;
  if constexpr (LDS) {
    // Eight rounds of loads in flight per thread.
    for (uint32_t j0 = 0; j0 < rounds; j0 += 8) {
      int32_t idx[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t p = (j0 + u) * kSubThreads + t;
        idx[u] = p < n ? srow[p] : -1;
      }
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (idx[u] >= 0 && (int64_t)idx[u] < N) ? row[idx[u]] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t p = (j0 + u) * kSubThreads + t;
        const bool ok = idx[u] >= 0 && (int64_t)idx[u] < N;
        const uint64_t m = __ballot(ok);
        if (p < n) s_keys[p] = order_key(v[u]);
        const uint32_t w0 = ((j0 + u) * kSubThreads + 64 * wave) / 32;  // this wave's 64 positions
        if ((j0 + u) < rounds && lane < 2) s_valid[w0 + lane] = (uint32_t)(m >> (32 * lane));
        nvalid += ok ? 1u : 0u;
      }
    }
    __syncthreads();
  } else {
    for (uint32_t p = t; p < n; p += kSubThreads) {
      const int32_t i = srow[p];
      nvalid += (i >= 0 && (int64_t)i < N) ? 1u : 0u;
    }
  }
  // (key, position) of every valid entry of this thread.
  auto each = [&](auto f) {
    for (uint32_t p = t; p < n; p += kSubThreads) {
      if constexpr (LDS) {
        if ((s_valid[p >> 5] >> (p & 31)) & 1u) f(make_uint2(s_keys[p], p));
      } else {
        uint32_t key;
        if (gather(p, key)) f(make_uint2(key, p));
      }
    }
  };

  uint32_t V;
  (void)block_exclusive_scan(nvalid, s_wtot, &V);
  const uint32_t k = (uint32_t)top_k < V ? (uint32_t)top_k : V;
  if (t == 0) n_out[b] = (int32_t)k;
  if (k == 0) return;
  uint32_t T = 0, last = 0xffffffffu;  // k == V: every valid entry is chosen
  if (k < V) radix_select<kSubThreads>(each, k, index_bits((int64_t)n), h, s_wtot, s_out, &T, &last);

  auto chosen_at = [&](uint32_t p) -> bool {
    if (p >= n) return false;
    uint32_t key;
    if constexpr (LDS) {
      if (!((s_valid[p >> 5] >> (p & 31)) & 1u)) return false;
      key = s_keys[p];
    } else {
      if (!gather(p, key)) return false;
    }
    return key > T || (key == T && p <= last);
  };
  int32_t* orow = out + (size_t)b * top_k;
  const uint64_t below_me = (1ull << lane) - 1ull;
  uint32_t base = 0;
  for (uint32_t g0 = 0; g0 < rounds; g0 += kSubGroupRounds) {
    const uint32_t gr = rounds - g0 < (uint32_t)kSubGroupRounds ? rounds - g0 : (uint32_t)kSubGroupRounds;
    for (uint32_t j = 0; j < gr; ++j) {
      const uint64_t m = __ballot(chosen_at((g0 + j) * kSubThreads + t));
      if (lane == 0) s_cnt[j * kSubWaves + wave] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    const uint32_t c = (uint32_t)t < gr * kSubWaves ? s_cnt[t] : 0u;
    uint32_t tot;
    const uint32_t off = block_exclusive_scan(c, s_wtot, &tot);
    if ((uint32_t)t < gr * kSubWaves) s_cnt[t] = off;
    __syncthreads();
    for (uint32_t j = 0; j < gr; ++j) {
      const uint32_t p = (g0 + j) * kSubThreads + t;
      const bool c = chosen_at(p);
      const uint64_t m = __ballot(c);
      if (c) orow[base + s_cnt[j * kSubWaves + wave] + (uint32_t)__popcll(m & below_me)] = srow[p];
    }
    base += tot;
    __syncthreads();  // s_cnt is rewritten by the next group
  }
}

}  // namespace

// Static LDS of the kernel (histograms, scan and compaction scratch, and the
// radix selection's own) kept out of the dynamic budget.
constexpr size_t kSubStaticLds = 24 * 1024;

// Keys (4 B per entry) and the bitmap, in whole rounds of 1024 positions.
size_t subset_lds_bytes(int32_t cap) { return 4 * (size_t)cap + 4 * 32 * (((size_t)cap + kSubThreads - 1) / kSubThreads); }

hipError_t init_select_topk_subset(int device, size_t* max_dynamic_lds) {
  int lds = 0;
  hipError_t e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, device);
  if (e != hipSuccess) return e;
  const size_t dyn = (size_t)lds > kSubStaticLds ? (size_t)lds - kSubStaticLds : 0;
  *max_dynamic_lds = dyn;
  return hipFuncSetAttribute((const void*)sel_subset_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)dyn);
}

hipError_t launch_select_topk_subset(const float* scores, int B, int64_t N, const int32_t* subset,
                                     const int32_t* n_subset, int32_t cap, int32_t top_k, int32_t* out,
                                     int32_t* n_out, size_t max_dynamic_lds, hipStream_t stream) {
  const size_t lds = subset_lds_bytes(cap);
  if (lds <= max_dynamic_lds)
    hipLaunchKernelGGL(sel_subset_kernel<true>, dim3(B), dim3(kSubThreads), lds, stream, scores, N, subset, n_subset,
                       cap, top_k, out, n_out);
  else
    hipLaunchKernelGGL(sel_subset_kernel<false>, dim3(B), dim3(kSubThreads), 0, stream, scores, N, subset, n_subset,
                       cap, top_k, out, n_out);
  return hipGetLastError();
}

}  // namespace fm
