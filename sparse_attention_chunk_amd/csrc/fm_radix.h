// Exact radix selection on order-preserving 32-bit keys, shared by the
// top-K kernels (fm_select.hip, fm_subset.hip): wave scans on DPP moves, the
// block-wide bin search over a kSelBins histogram, and the selection of the
// k-th largest key with ties broken towards the lowest index.
#pragma once

#include "fm_internal.h"

namespace fm {
namespace radix {

// Monotone map fp32 -> uint32: a < b (as floats, no NaN) iff key(a) < key(b).
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave64 inclusive prefix sum and max/min reductions on DPP lane moves
// (gfx9 family): row shifts by 1, 2, 4, 8 within each row of 16 lanes, then
// lane 15 of a row broadcast to the next row and lane 31 to the upper half.
// A lane with no source lane adds the identity (`old`).
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t identity, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
  return wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
// Reductions: the inclusive scan's last lane, read by every lane.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return __builtin_amdgcn_readlane(wave_prefix_sum(v), 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return __builtin_amdgcn_readlane(wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; }), 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return __builtin_amdgcn_readlane(wave_scan(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; }),
                                   63);
}

// Block-wide: the digit (bin) holding the k-th element (1-based) of a
// kSelBins-bin histogram, counting from the top bin down (largest) or from
// bin 0 up, the number of elements in the bins before it in that order, and
// the bin's own count (s_out[0..2]).  Thread t owns the PER consecutive bins
// from t PER (read as 16-byte vectors); prefix sums by a wave scan plus one
// step across the waves through LDS.  Ends with a barrier, after which every
// thread sees s_out.
template <int THREADS>
__device__ void block_find(const uint32_t* h, uint32_t k, uint32_t* s_wtot, uint32_t* s_out, bool largest) {
  constexpr int PER = kSelBins / THREADS;
  static_assert(PER == 2 || PER % 4 == 0, "bins per thread");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  uint32_t cnt[PER];
  if constexpr (PER == 2) {
    const uint2 v = *(const uint2*)(h + 2 * t);
    cnt[0] = v.x;
    cnt[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const uint4 v = *(const uint4*)(h + PER * t + 4 * q);
      cnt[4 * q] = v.x;
      cnt[4 * q + 1] = v.y;
      cnt[4 * q + 2] = v.z;
      cnt[4 * q + 3] = v.w;
    }
  }
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) tot += cnt[j];
  const uint32_t incl = wave_prefix_sum(tot);
  if (lane == 63) s_wtot[wave] = incl;
  __syncthreads();
  uint32_t below = 0, all = 0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) {
    const uint32_t v = s_wtot[w];
    below += w < wave ? v : 0u;
    all += v;
  }
  const uint32_t prefix_incl = below + incl;
  const uint32_t before = largest ? all - prefix_incl : prefix_incl - tot;
  if (before < k && k <= before + tot) {
    // This thread's bins hold the k-th element: walk them in order.
    uint32_t acc = before;
    bool found = false;
#pragma unroll
    for (int jj = 0; jj < PER; ++jj) {
      const int j = largest ? PER - 1 - jj : jj;
      if (!found && acc + cnt[j] >= k) {
        s_out[0] = (uint32_t)(t * PER + j);
        s_out[1] = acc;
        s_out[2] = cnt[j];
        found = true;
      }
      acc += cnt[j];
    }
  }
  __syncthreads();
}

// Zeroes a kSelBins histogram with 16-byte stores.
template <int THREADS>
__device__ __forceinline__ void clear_bins(uint32_t* h) {
#pragma unroll
  for (int i = 4 * (int)threadIdx.x; i < kSelBins; i += 4 * THREADS) *(uint4*)(h + i) = make_uint4(0, 0, 0, 0);
}

// Radix selection over a stream of (key, index) pairs produced by `each`
// (called once per pass with a functor taking a pair): the k-th largest key
// T (1-based k <= stream size) and the largest index kept among the keys
// equal to T when ties go to the lowest indices (0xffffffff when every key
// equal to T is kept).
//
// A first pass finds the smallest and largest key: their common high bits
// are every key's, so the digit passes (at most 11 bits each) start below
// them.  Concentrated keys (scores in a narrow range) would otherwise fall
// into a few bins of the first pass and serialise its LDS atomics.  The
// index passes cover the low idx_bits bits and run only when some key equal
// to T is left out.
template <int THREADS, typename Each>
__device__ void radix_select(Each each, uint32_t k, int idx_bits, uint32_t* h, uint32_t* s_wtot, uint32_t* s_out,
                             uint32_t* T_out, uint32_t* last_out) {
  __shared__ uint32_t s_mm[3 * (THREADS / 64)];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0u, cnt = 0u;
  each([&](uint2 e) {
    kmin = e.x < kmin ? e.x : kmin;
    kmax = e.x > kmax ? e.x : kmax;
    ++cnt;
  });
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  cnt = wave_sum_u32(cnt);
  if (lane == 0) {
    s_mm[3 * wave] = kmin;
    s_mm[3 * wave + 1] = kmax;
    s_mm[3 * wave + 2] = cnt;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
  cnt = 0u;
  for (int w = 0; w < THREADS / 64; ++w) {
    kmin = s_mm[3 * w] < kmin ? s_mm[3 * w] : kmin;
    kmax = s_mm[3 * w + 1] > kmax ? s_mm[3 * w + 1] : kmax;
    cnt += s_mm[3 * w + 2];
  }
  // lo = number of low key bits still open; prefix = the bits above them.
  // Two histogram buffers: a pass counts into one while the other is
  // cleared for the next pass.
  int lo = kmin == kmax ? 0 : 32 - __builtin_clz(kmin ^ kmax);
  uint64_t prefix = (uint64_t)kmax >> lo;
  uint32_t n_eq = cnt;  // keys equal to the prefix so far
  int buf = 0;
  clear_bins<THREADS>(h);
  __syncthreads();
  while (lo > 0) {
    const int w = lo >= 11 ? 11 : lo;
    const int shift = lo - w;
    const int nb = 1 << w;
    uint32_t* hb = h + buf * kSelBins;
    each([&](uint2 e) {
      if (((uint64_t)e.x >> lo) == prefix) atomicAdd(&hb[(e.x >> shift) & (nb - 1)], 1u);
    });
    clear_bins<THREADS>(h + (buf ^ 1) * kSelBins);
    __syncthreads();
    block_find<THREADS>(hb, k, s_wtot, s_out, true);
    prefix = (prefix << w) | s_out[0];
    k -= s_out[1];
    n_eq = s_out[2];
    lo = shift;
    buf ^= 1;
  }
  const uint32_t T = (uint32_t)prefix;  // k = keys equal to T still to keep (>= 1)
  *T_out = T;
  if (n_eq == k) {  // every key equal to T is kept
    *last_out = 0xffffffffu;
    return;
  }
  uint64_t iprefix = 0;
  lo = idx_bits;
  while (lo > 0) {
    const int w = lo >= 11 ? 11 : lo;
    const int shift = lo - w;
    const int nb = 1 << w;
    uint32_t* hb = h + buf * kSelBins;
    each([&](uint2 e) {
      if (e.x == T && ((uint64_t)e.y >> lo) == iprefix) atomicAdd(&hb[(e.y >> shift) & (nb - 1)], 1u);
    });
    clear_bins<THREADS>(h + (buf ^ 1) * kSelBins);
    __syncthreads();
    block_find<THREADS>(hb, k, s_wtot, s_out, false);
    iprefix = (iprefix << w) | s_out[0];
    k -= s_out[1];
    lo = shift;
    buf ^= 1;
  }
  *last_out = (uint32_t)iprefix;
}

// Bits needed for chunk indices below n (at least 1).
__device__ inline int index_bits(int64_t n) {
  const uint32_t m = n > 1 ? (uint32_t)(n - 1) : 1u;
  return 32 - __builtin_clz(m);
}

}  // namespace radix
}  // namespace fm
