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
// One block of 1024 threads per row selects; position p of the list is
// handled by thread p mod 1024 (coalesced list reads), in rounds of 1024
// positions.  Lists of up to 32 rounds keep their keys (order-preserving
// uint32 of the scores) and a validity bitmap in LDS: gathered beforehand by
// one block per round (sub_gather_kernel) when the workspace can stage them,
// else by the selecting block with every load in flight together.  Longer
// lists gather their keys again in every pass, eight rounds of loads at a
// time.  Lists in LDS longer than 8192 entries narrow the selection with a
// sampled cut-off (sampled_select: candidates above it, an exact radix
// selection among them, and the chosen ones written in list order through a
// bitmap of the list); otherwise an exact radix selection over the whole
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

constexpr int kSubLdsRounds = 32;  // lists of up to 32 x 1024 entries keep their keys in LDS
constexpr int kSubBatch = 8;        // rounds of loads in flight in the gathering variant
constexpr size_t kSubLdsBytes = (size_t)kSubLdsRounds * kSubThreads * 4 + kSubLdsRounds * kSubWaves * 8;

__device__ __forceinline__ bool in_range(int32_t i, int64_t N) { return i >= 0 && (int64_t)i < N; }

// Keys of a list held in LDS, gathered beforehand by many blocks (the
// gathers are random reads, which one block per row issues too slowly):
// per row, kSubLdsRounds x 1024 keys then the validity bitmap (32 words per
// round), in the workspace's staging rows.
constexpr size_t kSubPreRow = (size_t)kSubLdsRounds * kSubThreads + (size_t)kSubLdsRounds * 2 * kSubWaves;
static_assert(kSubPreRow <= kSubStageRowWords, "staging row size");

// grid = (rounds, B), 256 threads: round r of row b, positions r 1024 + 256 u
// + t (u = 0..3).  Writes each position's key and the round's bitmap words.
__global__ __launch_bounds__(256) void sub_gather_kernel(const float* __restrict__ scores, int64_t N,
                                                         const int32_t* __restrict__ subset,
                                                         const int32_t* __restrict__ n_subset, int32_t cap,
                                                         uint32_t* __restrict__ pre) {
  const int b = blockIdx.y;
  const uint32_t r = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t n64 = n_subset ? (int64_t)n_subset[b] : (int64_t)cap;
  const uint32_t n = (uint32_t)(n64 < 0 ? 0 : (n64 > cap ? cap : n64));
  if (r * kSubThreads >= n) return;
  const int32_t* srow = subset + (size_t)b * cap;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)srow, 0, (int)(4 * n), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scores + (size_t)b * N), 0, (int)(N < 0x20000000 ? 4 * N : 0x7fffffff), 0x00020000);
  uint32_t* keys = pre + (size_t)b * kSubPreRow;
  uint32_t* bits = keys + (size_t)kSubLdsRounds * kSubThreads;
  int32_t idx[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) idx[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * (r * kSubThreads + 256 * u + t), 0, 0);
  uint32_t v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t p = r * kSubThreads + 256 * u + t;
    if (!(p < n && in_range(idx[u], N))) idx[u] = -1;
    v[u] = __builtin_amdgcn_raw_buffer_load_b32(rv, idx[u] >= 0 ? 4u * (uint32_t)idx[u] : 0x80000000u, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t p = r * kSubThreads + 256 * u + t;
    keys[p] = order_key(__uint_as_float(v[u]));
    const uint64_t m = __ballot(idx[u] >= 0);
    if (lane < 2) bits[(p - lane) / 32 + lane] = (uint32_t)(m >> (32 * lane));  // words of this wave's 64 positions
  }
}

constexpr uint32_t kSubSample = 4096;      // sampled keys for the cut-off
constexpr uint32_t kSubCandMax = 16384;    // candidates compacted into the first half of the key area

// The selection of a long list held in LDS, narrowed by a sample (as the row
// top-K does): the m-th largest of 4096 evenly spaced valid keys gives a
// cut-off L with m chosen so that about k plus four standard deviations of
// the list's keys are expected at or above L.  One pass over the list keeps
// the keys >= L in registers and writes them, at each thread's offset from a
// block scan of the counts, into the first half of the key area (keys) and
// the second half (positions): unordered, since the exact radix selection
// that then runs over these candidates does not depend on their order.  The
// chosen ones set their bits in a bitmap of the list (over the validity
// bitmap, no longer needed), and a scan of its words writes them in list
// order.  Returns false, with LDS untouched, when the candidates are fewer
// than k or too many; the caller then selects over the whole list.
__device__ __forceinline__ bool sampled_select(uint32_t* s_keys, uint32_t* s_valid, uint32_t n, uint32_t rounds,
                                               uint32_t V, uint32_t k, const int32_t* srow, int32_t* orow,
                                               uint32_t* h, uint32_t* s_wtot, uint32_t* s_out) {
  const int t = threadIdx.x;
  auto valid_at = [&](uint32_t p) { return (s_valid[p >> 5] >> (p & 31)) & 1u; };

  // 1. Cut-off from the sample (sample i at position i n / 4096).
  constexpr int kPer = kSubSample / kSubThreads;
  uint32_t sk[kPer];
  uint32_t sv = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const uint32_t i = (uint32_t)t + kSubThreads * u;
    const uint32_t p = (uint32_t)(((uint64_t)i * n) / kSubSample);
    sk[u] = s_keys[p];
    sv |= valid_at(p) << u;
  }
  uint32_t S;
  (void)block_exclusive_scan((uint32_t)__popc(sv), s_wtot, &S);
  if (S == 0) return false;
  const double expect = (double)k * (double)S / (double)V;
  const double mm = ceil(expect + 4.0 * sqrt(expect) + 16.0);
  const uint32_t m = mm >= (double)S ? S : (uint32_t)mm;
  uint32_t L, unused;
  radix_select<kSubThreads, false>(
      [&](auto f) {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          if ((sv >> u) & 1u) f(make_uint2(sk[u], (uint32_t)t + kSubThreads * u));
      },
      m, 0, h, s_wtot, s_out, &L, &unused);

  // 2. Candidates (keys >= L) of this thread, in registers (the key area is
  // overwritten below); the scan's barriers order every read before the
  // first write.  Every round's key and bitmap word is read (past the list
  // they are stale and masked off by p < n), so nothing here branches.
  uint32_t ck[kSubLdsRounds];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kSubLdsRounds; ++j) {
    const uint32_t p = (uint32_t)j * kSubThreads + t;
    ck[j] = s_keys[p];
    const uint32_t c = (uint32_t)(p < n) & valid_at(p) & (uint32_t)(ck[j] >= L);  // no short circuit
    mine |= c << j;
  }
  uint32_t C;
  uint32_t slot = block_exclusive_scan((uint32_t)__popc(mine), s_wtot, &C);
  if (C < k || C > kSubCandMax) return false;  // block-uniform; LDS untouched
  uint32_t* c_key = s_keys;
  uint32_t* c_pos = s_keys + kSubCandMax;
#pragma unroll
  for (int j = 0; j < kSubLdsRounds; ++j) {
    if ((mine >> j) & 1u) {
      c_key[slot] = ck[j];
      c_pos[slot] = (uint32_t)j * kSubThreads + t;
      ++slot;
    }
  }
  __syncthreads();
  // 3. Exact selection over the candidates (ties by list position).
  auto cand_each = [&](auto f) {
    for (uint32_t sl = t; sl < C; sl += kSubThreads) f(make_uint2(c_key[sl], c_pos[sl]));
  };
  uint32_t T, last;
  radix_select<kSubThreads>(cand_each, k, index_bits((int64_t)n), h, s_wtot, s_out, &T, &last);
  // 4. The chosen ones in list order: bit p % 32 of word p / 32 of the list
  // bitmap; thread t owns word t (positions 32 t .. 32 t + 31).
  const uint32_t words = rounds * (kSubThreads / 32);  // at most kSubThreads
  if ((uint32_t)t < words) s_valid[t] = 0u;
  __syncthreads();
  cand_each([&](uint2 e) {
    if (e.x > T || (e.x == T && e.y <= last)) atomicOr(&s_valid[e.y >> 5], 1u << (e.y & 31));
  });
  __syncthreads();
  uint32_t bits = (uint32_t)t < words ? s_valid[t] : 0u;
  uint32_t tot;
  uint32_t out_slot = block_exclusive_scan((uint32_t)__popc(bits), s_wtot, &tot);
  while (bits) {
    const uint32_t p = 32u * (uint32_t)t + (uint32_t)__builtin_ctz(bits);
    bits &= bits - 1u;
    orow[out_slot++] = srow[p];
  }
  return true;
}

// LDS: the list has at most kSubLdsRounds rounds; keys and the validity
// bitmap (bit p % 32 of word p / 32) live in dynamic LDS (kSubLdsBytes).
// PRE (with LDS): the keys and bitmap were gathered by sub_gather_kernel
// into pre; they are copied to LDS with coalesced reads.
template <bool LDS, bool PRE = false>
__global__ __launch_bounds__(kSubThreads) void sel_subset_kernel(const float* __restrict__ scores, int64_t N,
                                                                 const int32_t* __restrict__ subset,
                                                                 const int32_t* __restrict__ n_subset, int32_t cap,
                                                                 int32_t top_k, int32_t* __restrict__ out,
                                                                 int32_t* __restrict__ n_out,
                                                                 const uint32_t* __restrict__ pre) {
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
  uint32_t* s_valid = s_keys + (size_t)kSubLdsRounds * kSubThreads;

  uint32_t nvalid = 0;
  if constexpr (LDS && PRE) {
    const uint32_t* keys = pre + (size_t)b * kSubPreRow;
    const uint32_t* bits = keys + (size_t)kSubLdsRounds * kSubThreads;
    uint32_t v[kSubLdsRounds];
#pragma unroll
    for (int j = 0; j < kSubLdsRounds; ++j)
      if ((uint32_t)j < rounds) v[j] = keys[(uint32_t)j * kSubThreads + t];
    const uint32_t word = (uint32_t)t < rounds * 2 * kSubWaves ? bits[t] : 0u;
#pragma unroll
    for (int j = 0; j < kSubLdsRounds; ++j)
      if ((uint32_t)j < rounds) s_keys[(uint32_t)j * kSubThreads + t] = v[j];
    if ((uint32_t)t < rounds * 2 * kSubWaves) s_valid[t] = word;
    nvalid = (uint32_t)__popc(word);
    __syncthreads();
  } else if constexpr (LDS) {
    // Every load in flight before the first use, through range-checked
    // buffer views: reads past the list or the row return 0, no branch.
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)srow, 0, (int)(4 * n), 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)row, 0, (int)(N < 0x20000000 ? 4 * N : 0x7fffffff), 0x00020000);
    int32_t idx[kSubLdsRounds];
#pragma unroll
    for (int j = 0; j < kSubLdsRounds; ++j)
      idx[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * ((uint32_t)j * kSubThreads + t), 0, 0);
    uint32_t v[kSubLdsRounds];
#pragma unroll
    for (int j = 0; j < kSubLdsRounds; ++j) {
      const uint32_t p = (uint32_t)j * kSubThreads + t;
      if (!(p < n && in_range(idx[j], N))) idx[j] = -1;
      v[j] = __builtin_amdgcn_raw_buffer_load_b32(rv, idx[j] >= 0 ? 4u * (uint32_t)idx[j] : 0x80000000u, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kSubLdsRounds; ++j) {
      if ((uint32_t)j < rounds) {
        const bool ok = idx[j] >= 0;
        const uint64_t m = __ballot(ok);
        s_keys[(uint32_t)j * kSubThreads + t] = order_key(__uint_as_float(v[j]));
        if (lane < 2) s_valid[j * 2 * kSubWaves + 2 * wave + lane] = (uint32_t)(m >> (32 * lane));
        nvalid += ok ? 1u : 0u;
      }
    }
    __syncthreads();
  } else {
    for (uint32_t p = t; p < n; p += kSubThreads) nvalid += in_range(srow[p], N) ? 1u : 0u;
  }
  // fn(key, position) for each of this thread's valid entries.
  auto each_entry = [&](auto fn) {
    if constexpr (LDS) {
      for (uint32_t j0 = 0; j0 < rounds; j0 += 4) {
        uint32_t kk[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t p = (j0 + u) * kSubThreads + t;
          ok[u] = j0 + u < rounds && ((s_valid[p >> 5] >> (p & 31)) & 1u);
          kk[u] = s_keys[p];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (ok[u]) fn(kk[u], (j0 + u) * kSubThreads + t);
      }
    } else {
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
  if constexpr (LDS) {
    if (k < V && n > 2 * kSubSample && sampled_select(s_keys, s_valid, n, rounds, V, k, srow, orow, h, s_wtot,
                                                      s_out))
      return;
  }
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

hipError_t init_select_topk_subset() {
  hipError_t e = hipFuncSetAttribute((const void*)sel_subset_kernel<true, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSubLdsBytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)sel_subset_kernel<true, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)kSubLdsBytes);
}

hipError_t launch_select_topk_subset(const Workspace& ws, const float* scores, int B, int64_t N,
                                     const int32_t* subset, const int32_t* n_subset, int32_t cap, int32_t top_k,
                                     int32_t* out, int32_t* n_out, hipStream_t stream) {
  if (cap <= kSubFastCap) return launch_select_topk_subset_fast(ws, scores, B, N, subset, n_subset, cap, top_k, out,
                                                                 n_out, stream);
  if (cap <= kSubLdsRounds * kSubThreads) {
    uint32_t* pre = ws.sub_stage;
    if (B > 0 && cap > 0) {
      const dim3 grid((unsigned)((cap + kSubThreads - 1) / kSubThreads), (unsigned)B);
      hipLaunchKernelGGL(sub_gather_kernel, grid, dim3(256), 0, stream, scores, N, subset, n_subset, cap, pre);
      hipLaunchKernelGGL((sel_subset_kernel<true, true>), dim3(B), dim3(kSubThreads), kSubLdsBytes, stream, scores, N,
                         subset, n_subset, cap, top_k, out, n_out, (const uint32_t*)pre);
    } else {
      hipLaunchKernelGGL((sel_subset_kernel<true, false>), dim3(B), dim3(kSubThreads), kSubLdsBytes, stream, scores,
                         N, subset, n_subset, cap, top_k, out, n_out, (const uint32_t*)nullptr);
    }
  } else {
    hipLaunchKernelGGL((sel_subset_kernel<false, false>), dim3(B), dim3(kSubThreads), 0, stream, scores, N, subset,
                       n_subset, cap, top_k, out, n_out, (const uint32_t*)nullptr);
  }
  return hipGetLastError();
}

}  // namespace fm
