// Keep masks (FlashMemory DS-V4 Retriever README, "Usage": select_topk with
// top_k=... or threshold=...; "Inference flow": keep_mask = top-K of the
// scores, or sigmoid > thresh).
//
// Top-K is an exact per-row radix select on order-preserving 32-bit keys of
// the fp32 scores: three digit passes (11, 11, 10 bits) find the K-th
// largest key T and how many keys equal to T still fit (k_eq); ties at T go
// to the lowest chunk indices, which makes the mask unique.  The final pass
// counts keys equal to T per block, and each block ranks its own equal keys
// after the counts of the blocks before it.  All passes stream the row's
// scores (4 bytes per chunk); the mask is written once (1 byte per chunk).
#include "fm_internal.h"

namespace fm {
namespace {

// Monotone map fp32 -> uint32: a < b (as floats, no NaN) iff key(a) < key(b).
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int64_t row_valid(const int32_t* valid_n, int b, int64_t N) {
  if (!valid_n) return N;
  const int64_t v = valid_n[b];
  return v < 0 ? 0 : (v > N ? N : v);
}

// state[b] = {prefix, k_remaining, mode, unused}; mode 0 = select, 1 = keep
// every valid chunk, 2 = keep none.
enum : uint32_t { kSelect = 0, kKeepAll = 1, kKeepNone = 2 };

__global__ void sel_init_kernel(const int32_t* valid_n, int64_t N, int32_t top_k, uint32_t* state, uint32_t* hist) {
  const int b = blockIdx.x;
  const int64_t vn = row_valid(valid_n, b, N);
  if (threadIdx.x == 0) {
    uint32_t mode = kSelect;
    if (top_k == 0 || vn == 0) mode = kKeepNone;
    else if ((int64_t)top_k >= vn) mode = kKeepAll;
    state[4 * b + 0] = 0;
    state[4 * b + 1] = (uint32_t)top_k;
    state[4 * b + 2] = mode;
    state[4 * b + 3] = 0;
  }
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) hist[(size_t)b * kSelBins + i] = 0;
}

// Digit pass: histogram of digit `pass` over keys whose higher digits equal
// the prefix found so far.  grid = (blocks per row, B).
__global__ __launch_bounds__(kSelThreads) void sel_hist_kernel(const float* scores, int64_t N,
                                                               const int32_t* valid_n, int pass,
                                                               const uint32_t* state, uint32_t* hist) {
  const int b = blockIdx.y;
  if (state[4 * b + 2] != kSelect) return;
  __shared__ uint32_t h[kSelBins];
  for (int i = threadIdx.x; i < kSelBins; i += kSelThreads) h[i] = 0;
  __syncthreads();
  const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
  const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
  const int hi_shift = pass == 0 ? 32 : (pass == 1 ? 21 : 10);
  const uint32_t prefix = state[4 * b + 0];
  const int64_t vn = row_valid(valid_n, b, N);
  const int64_t base = (int64_t)blockIdx.x * kSelSlice;
  const float* row = scores + (size_t)b * N;
  for (int it = 0; it < kSelItems; ++it) {
    const int64_t n = base + (int64_t)it * kSelThreads + threadIdx.x;
    if (n < vn) {
      const uint32_t key = order_key(row[n]);
      if (hi_shift == 32 || (key >> hi_shift) == prefix) atomicAdd(&h[(key >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kSelBins; i += kSelThreads)
    if (h[i]) atomicAdd(&hist[(size_t)b * kSelBins + i], h[i]);
}

// One block per row: the digit of the k-th largest key among the candidates.
// Thread t owns bins [8t, 8t + 8); a suffix sum over threads gives each
// thread the count of candidates in higher bins.
__global__ __launch_bounds__(kSelThreads) void sel_find_kernel(int pass, uint32_t* state, uint32_t* hist) {
  const int b = blockIdx.x;
  if (state[4 * b + 2] != kSelect) return;
  const int nbins = pass == 2 ? 1024 : 2048;
  const int per = nbins / kSelThreads;  // 8 or 4
  uint32_t* hb = hist + (size_t)b * kSelBins;
  uint32_t cnt[8];
  uint32_t tot = 0;
  for (int j = 0; j < per; ++j) {
    cnt[j] = hb[threadIdx.x * per + j];
    tot += cnt[j];
  }
  __shared__ uint32_t sums[kSelThreads];
  sums[threadIdx.x] = tot;
  __syncthreads();
  // inclusive suffix scan: above[t] = sum over t' > t
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const uint32_t v = threadIdx.x + off < kSelThreads ? sums[threadIdx.x + off] : 0u;
    __syncthreads();
    sums[threadIdx.x] += v;
    __syncthreads();
  }
  const uint32_t incl = sums[threadIdx.x];
  const uint32_t above = incl - tot;
  const uint32_t k_rem = state[4 * b + 1];
  __syncthreads();
  if (above < k_rem && k_rem <= incl) {
    uint32_t acc = above;
    for (int j = per - 1; j >= 0; --j) {
      if (acc + cnt[j] >= k_rem) {
        const uint32_t digit = (uint32_t)(threadIdx.x * per + j);
        const int bits = pass == 2 ? 10 : 11;
        state[4 * b + 0] = (state[4 * b + 0] << bits) | digit;
        state[4 * b + 1] = k_rem - acc;
        break;
      }
      acc += cnt[j];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kSelBins; i += kSelThreads) hb[i] = 0;
}

// Count of keys equal to T per block.
__global__ __launch_bounds__(kSelThreads) void sel_count_eq_kernel(const float* scores, int64_t N,
                                                                   const int32_t* valid_n, const uint32_t* state,
                                                                   uint32_t* eq, int blocks_per_row) {
  const int b = blockIdx.y;
  if (state[4 * b + 2] != kSelect) return;
  const uint32_t T = state[4 * b + 0];
  const int64_t vn = row_valid(valid_n, b, N);
  const int64_t base = (int64_t)blockIdx.x * kSelSlice;
  const float* row = scores + (size_t)b * N;
  uint32_t c = 0;
  for (int it = 0; it < kSelItems; ++it) {
    const int64_t n = base + (int64_t)it * kSelThreads + threadIdx.x;
    if (n < vn && order_key(row[n]) == T) ++c;
  }
  __shared__ uint32_t red[kSelThreads];
  red[threadIdx.x] = c;
  __syncthreads();
  for (int off = kSelThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) eq[(size_t)b * blocks_per_row + blockIdx.x] = red[0];
}

// Mask: key > T, or key == T with row rank among the equal keys < k_eq.
// Thread t handles kSelItems consecutive chunks, so an exclusive scan over
// threads of their equal counts ranks the block's equal keys in index order.
__global__ __launch_bounds__(kSelThreads) void sel_mask_kernel(const float* scores, int64_t N,
                                                               const int32_t* valid_n, const uint32_t* state,
                                                               const uint32_t* eq, int blocks_per_row,
                                                               uint8_t* mask) {
  const int b = blockIdx.y;
  const uint32_t mode = state[4 * b + 2];
  const uint32_t T = state[4 * b + 0];
  const uint32_t k_eq = state[4 * b + 1];
  const int64_t vn = row_valid(valid_n, b, N);
  const int64_t n0 = (int64_t)blockIdx.x * kSelSlice + (int64_t)threadIdx.x * kSelItems;
  const float* row = scores + (size_t)b * N;
  uint8_t* mrow = mask + (size_t)b * N;

  __shared__ uint32_t sums[kSelThreads];
  __shared__ uint32_t s_base;
  uint32_t keys[kSelItems];
  uint32_t mine = 0;
  if (mode == kSelect) {
    for (int j = 0; j < kSelItems; ++j) {
      const int64_t n = n0 + j;
      keys[j] = n < vn ? order_key(row[n]) : 0u;
      mine += (n < vn && keys[j] == T) ? 1u : 0u;
    }
    if (threadIdx.x == 0) {
      uint32_t s = 0;
      for (int i = 0; i < (int)blockIdx.x; ++i) s += eq[(size_t)b * blocks_per_row + i];
      s_base = s;
    }
    sums[threadIdx.x] = mine;
    __syncthreads();
    for (int off = 1; off < kSelThreads; off <<= 1) {  // inclusive prefix scan
      const uint32_t v = threadIdx.x >= (unsigned)off ? sums[threadIdx.x - off] : 0u;
      __syncthreads();
      sums[threadIdx.x] += v;
      __syncthreads();
    }
  }
  uint32_t rank = mode == kSelect ? s_base + sums[threadIdx.x] - mine : 0u;
  for (int j = 0; j < kSelItems; ++j) {
    const int64_t n = n0 + j;
    if (n >= N) break;
    uint8_t m = 0;
    if (n < vn) {
      if (mode == kKeepAll) {
        m = 1;
      } else if (mode == kSelect) {
        if (keys[j] > T) {
          m = 1;
        } else if (keys[j] == T) {
          m = rank < k_eq ? 1 : 0;
          ++rank;
        }
      }
    }
    mrow[n] = m;
  }
}

__global__ __launch_bounds__(256) void threshold_kernel(const float* scores, int64_t N, const int32_t* valid_n,
                                                        float threshold, uint8_t* mask) {
  const int b = blockIdx.y;
  const int64_t vn = row_valid(valid_n, b, N);
  const float* row = scores + (size_t)b * N;
  uint8_t* mrow = mask + (size_t)b * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < N; n += stride)
    mrow[n] = (n < vn && row[n] > threshold) ? 1 : 0;
}

}  // namespace

hipError_t launch_select_topk(const Workspace& ws, const float* scores, int B, int64_t N, const int32_t* valid_n,
                              int32_t top_k, uint8_t* mask, hipStream_t stream) {
  const int blocks_per_row = (int)((N + kSelSlice - 1) / kSelSlice);
  hipLaunchKernelGGL(sel_init_kernel, dim3(B), dim3(256), 0, stream, valid_n, N, top_k, ws.sel_state, ws.sel_hist);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(sel_hist_kernel, dim3(blocks_per_row, B), dim3(kSelThreads), 0, stream, scores, N, valid_n,
                       pass, (const uint32_t*)ws.sel_state, ws.sel_hist);
    hipLaunchKernelGGL(sel_find_kernel, dim3(B), dim3(kSelThreads), 0, stream, pass, ws.sel_state, ws.sel_hist);
  }
  hipLaunchKernelGGL(sel_count_eq_kernel, dim3(blocks_per_row, B), dim3(kSelThreads), 0, stream, scores, N, valid_n,
                     (const uint32_t*)ws.sel_state, ws.sel_eq, blocks_per_row);
  hipLaunchKernelGGL(sel_mask_kernel, dim3(blocks_per_row, B), dim3(kSelThreads), 0, stream, scores, N, valid_n,
                     (const uint32_t*)ws.sel_state, (const uint32_t*)ws.sel_eq, blocks_per_row, mask);
  return hipGetLastError();
}

hipError_t launch_select_threshold(const float* scores, int B, int64_t N, const int32_t* valid_n, float threshold,
                                   uint8_t* mask, hipStream_t stream) {
  const int64_t per_block = 256 * 16;
  const unsigned gx = (unsigned)((N + per_block - 1) / per_block);
  hipLaunchKernelGGL(threshold_kernel, dim3(gx, B), dim3(256), 0, stream, scores, N, valid_n, threshold, mask);
  return hipGetLastError();
}

}  // namespace fm
