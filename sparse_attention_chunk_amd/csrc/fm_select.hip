// Keep masks (FlashMemory DS-V4 Retriever README, "Usage": select_topk with
// top_k=... or threshold=...; "Inference flow": keep_mask = top-K of the
// scores, or sigmoid > thresh).
//
// Top-K is an exact per-row selection on order-preserving 32-bit keys of the
// fp32 scores; ties at the K-th key go to the lowest chunk indices, which
// makes the mask unique.  Three kernels per call:
//   1. sample: one block per row reads 8192 keys (64 runs of 128 chunks
//      spread over the row; the whole row when it is shorter) and picks a
//      cut-off L, the m-th largest sampled key, with m chosen so that about
//      K plus four standard deviations of the row's keys are expected at or
//      above L (a row that fits in the sample gets its exact K-th key);
//   2. collect: one pass over the row writes the mask (0 everywhere, 1 for
//      every valid chunk when K keeps them all) and writes the (key, index)
//      pairs of keys >= L to the row's candidate list, one region per block;
//   3. final: one block per row selects exactly among the candidates: radix
//      passes over the key give the K-th largest key T and how many keys equal
//      to T are kept, radix passes over the index of the keys equal to T give
//      the last index kept; those candidates' mask bytes are set.  When fewer
//      than K keys reached L (the sample was unrepresentative), the same
//      passes run over the whole row instead, so the result is always exact.
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

// state[b] = {cut-off L, unused, mode, unused}
enum : uint32_t { kSelect = 0, kKeepAll = 1, kKeepNone = 2 };

constexpr int kSampleRuns = 64;
constexpr int kSampleRun = 128;
constexpr int kSampleSize = kSampleRuns * kSampleRun;  // 8192
constexpr int kSampleThreads = 1024;
constexpr int kSamplePerThread = kSampleSize / kSampleThreads;  // 8

// Block-wide: the digit (bin) holding the k-th element (1-based) of a
// histogram, counting from the top bin down (largest) or from bin 0 up, and
// the number of elements in the bins before it in that order.  Thread t owns
// bins [t per, t per + per); prefix sums by wave shuffles plus one step
// across the waves through LDS.
template <int THREADS>
__device__ void block_find(const uint32_t* h, int nbins, uint32_t k, uint32_t* s_wtot, uint32_t* s_out,
                           bool largest) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int per = (nbins + THREADS - 1) / THREADS;
  const int owners = nbins / per;
  uint32_t cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t tot = 0;
  if (t < owners)
    for (int j = 0; j < per; ++j) {
      cnt[j] = h[t * per + j];
      tot += cnt[j];
    }
  uint32_t incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wtot[wave] = incl;
  __syncthreads();
  uint32_t below = 0, all = 0;
  for (int w = 0; w < THREADS / 64; ++w) {
    const uint32_t v = s_wtot[w];
    below += w < wave ? v : 0u;
    all += v;
  }
  const uint32_t prefix_incl = below + incl;
  const uint32_t before = largest ? all - prefix_incl : prefix_incl - tot;
  if (t < owners && before < k && k <= before + tot) {
    uint32_t acc = before;
    for (int jj = 0; jj < per; ++jj) {
      const int j = largest ? per - 1 - jj : jj;
      if (acc + cnt[j] >= k) {
        s_out[0] = (uint32_t)(t * per + j);
        s_out[1] = acc;
        break;
      }
      acc += cnt[j];
    }
  }
  __syncthreads();
}

// Radix selection over a stream of (key, index) pairs produced by `each`
// (called once per pass with a functor taking a pair): the k-th largest key
// T (1-based k <= stream size) and the largest index kept among the keys
// equal to T when ties go to the lowest indices.  Digit passes: key bits
// 31..21, 20..10, 9..0, then the same over the index of keys equal to T.
template <int THREADS, bool WITH_INDEX = true, typename Each>
__device__ void radix_select(Each each, uint32_t k, uint32_t* h, uint32_t* s_wtot, uint32_t* s_out, uint32_t* T_out,
                             uint32_t* last_out) {
  uint32_t prefix = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    const int hi = pass == 0 ? 32 : (pass == 1 ? 21 : 10);
    for (int i = threadIdx.x; i < kSelBins; i += THREADS) h[i] = 0;
    __syncthreads();
    each([&](uint2 e) {
      if (hi == 32 || (e.x >> hi) == prefix) atomicAdd(&h[(e.x >> shift) & (nb - 1)], 1u);
    });
    __syncthreads();
    block_find<THREADS>(h, nb, k, s_wtot, s_out, true);
    prefix = (prefix << (pass == 2 ? 10 : 11)) | s_out[0];
    k -= s_out[1];
    __syncthreads();
  }
  const uint32_t T = prefix;  // k = keys equal to T still to keep (>= 1)
  *T_out = T;
  if (!WITH_INDEX) return;
  uint32_t iprefix = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    const int hi = pass == 0 ? 32 : (pass == 1 ? 21 : 10);
    for (int i = threadIdx.x; i < kSelBins; i += THREADS) h[i] = 0;
    __syncthreads();
    each([&](uint2 e) {
      if (e.x == T && (hi == 32 || (e.y >> hi) == iprefix)) atomicAdd(&h[(e.y >> shift) & (nb - 1)], 1u);
    });
    __syncthreads();
    block_find<THREADS>(h, nb, k, s_wtot, s_out, false);
    iprefix = (iprefix << (pass == 2 ? 10 : 11)) | s_out[0];
    k -= s_out[1];
    __syncthreads();
  }
  *last_out = iprefix;
}

// 1. Cut-off per row from a sample.  grid = B, block = kSampleThreads.
__global__ __launch_bounds__(kSampleThreads) void sel_sample_kernel(const float* scores, int64_t N,
                                                                    const int32_t* valid_n, int32_t top_k,
                                                                    uint32_t* state) {
  const int b = blockIdx.x;
  const int64_t vn = row_valid(valid_n, b, N);
  uint32_t mode = kSelect;
  if (top_k == 0 || vn == 0) mode = kKeepNone;
  else if ((int64_t)top_k >= vn) mode = kKeepAll;
  if (mode != kSelect) {
    if (threadIdx.x == 0) {
      state[4 * b + 0] = 0;
      state[4 * b + 2] = mode;
    }
    return;
  }
  __shared__ uint32_t s_keys[kSampleSize];
  __shared__ uint32_t h[kSelBins];
  __shared__ uint32_t s_wtot[kSampleThreads / 64];
  __shared__ uint32_t s_out[2];
  const float* row = scores + (size_t)b * N;
  const bool whole = vn <= kSampleSize;
  const uint32_t S = whole ? (uint32_t)vn : (uint32_t)kSampleSize;
  // Sample i = t + kSampleThreads * j sits in run r = i / kSampleRun at
  // offset t % kSampleRun; run r starts at r (vn - kSampleRun) / 63.  All
  // loads are issued before the first LDS store.
  const int t = threadIdx.x;
  float v[kSamplePerThread];
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) {
    const uint32_t i = (uint32_t)t + kSampleThreads * j;
    int64_t n = i;
    if (!whole) {
      const int64_t r = (int64_t)(i / kSampleRun);
      n = r * (vn - kSampleRun) / (kSampleRuns - 1) + (i % kSampleRun);
    }
    v[j] = i < S ? row[n] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) {
    const uint32_t i = (uint32_t)t + kSampleThreads * j;
    if (i < S) s_keys[i] = order_key(v[j]);
  }
  __syncthreads();
  uint32_t m;
  if (whole) {
    m = (uint32_t)top_k;  // the sample is the row: its K-th key exactly
  } else {
    const double expect = (double)top_k * (double)S / (double)vn;
    const double mm = ceil(expect + 4.0 * sqrt(expect) + 16.0);
    m = mm >= (double)S ? S : (uint32_t)mm;
  }
  uint32_t L, unused;
  radix_select<kSampleThreads, false>(
      [&](auto f) {
        for (uint32_t i = threadIdx.x; i < S; i += kSampleThreads) f(make_uint2(s_keys[i], i));
      },
      m, h, s_wtot, s_out, &L, &unused);
  if (threadIdx.x == 0) {
    state[4 * b + 0] = L;
    state[4 * b + 2] = mode;
  }
}

// 2. Mask and candidates.  grid = (blocks per row, B); thread t handles
// kSelItems consecutive chunks.
__global__ __launch_bounds__(kSelThreads) void sel_collect_kernel(const float* scores, int64_t N,
                                                                  const int32_t* valid_n, const uint32_t* state,
                                                                  uint2* cand, uint32_t* cand_count, uint8_t* mask) {
  const int b = blockIdx.y;
  const uint32_t L = state[4 * b + 0];
  const uint32_t mode = state[4 * b + 2];
  const int64_t vn = row_valid(valid_n, b, N);
  const int64_t n0 = (int64_t)blockIdx.x * kSelSlice + (int64_t)threadIdx.x * kSelItems;
  const float* row = scores + (size_t)b * N;
  uint8_t* mrow = mask + (size_t)b * N;
  // Candidates of this block go to its own region of the row's list (the
  // region has room for the whole slice), counted without atomics.
  uint2* crow = cand + (size_t)b * N + (size_t)blockIdx.x * kSelSlice;

  const uint8_t keep = mode == kKeepAll ? 1 : 0;
  uint32_t ck[kSelItems];
  uint32_t is_cand = 0;  // bit j: chunk n0 + j is a candidate
  const bool full = n0 + kSelItems <= vn && ((((uintptr_t)(row + n0)) & 15) == 0);
  if (full) {
#pragma unroll
    for (int q = 0; q < kSelItems / 4; ++q) {
      const float4 v = *(const float4*)(row + n0 + 4 * q);
      const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * q + e;
        ck[j] = order_key(f[e]);
        if (mode == kSelect && ck[j] >= L) is_cand |= 1u << j;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
      const int64_t n = n0 + j;
      ck[j] = 0;
      if (n < vn) {
        ck[j] = order_key(row[n]);
        if (mode == kSelect && ck[j] >= L) is_cand |= 1u << j;
      }
    }
  }
  // Mask bytes: one 16-byte store when the run is whole, valid and aligned.
  if (n0 + kSelItems <= vn && ((((uintptr_t)(mrow + n0)) & 15) == 0)) {
    const uint32_t w = keep * 0x01010101u;
    *(uint4*)(mrow + n0) = make_uint4(w, w, w, w);
  } else {
    for (int j = 0; j < kSelItems && n0 + j < N; ++j) mrow[n0 + j] = n0 + j < vn ? keep : 0;
  }
  // Candidates at each thread's prefix within the block.
  __shared__ uint32_t s_wave[kSelThreads / 64];
  const uint32_t mine = __popc(is_cand);
  uint32_t incl = mine;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    before += w < wave ? s_wave[w] : 0u;
    tot += s_wave[w];
  }
  if (threadIdx.x == 0) cand_count[(size_t)b * gridDim.x + blockIdx.x] = tot;
  uint32_t pos = before + incl - mine;
#pragma unroll
  for (int j = 0; j < kSelItems; ++j) {  // static indices keep ck[] in registers
    if (is_cand & (1u << j)) crow[pos++] = make_uint2(ck[j], (uint32_t)(n0 + j));
  }
}

// 3. Exact selection among the candidates (or the whole row).  grid = B.
constexpr int kFinThreads = 1024;
constexpr int kFinLds = 8192;  // candidates staged in LDS; more are read from their regions each pass

__global__ __launch_bounds__(kFinThreads) void sel_final_kernel(const float* scores, int64_t N,
                                                                const int32_t* valid_n, int blocks_per_row,
                                                                int32_t top_k, const uint32_t* state,
                                                                const uint2* cand, const uint32_t* cand_count,
                                                                uint8_t* mask) {
  const int b = blockIdx.x;
  if (state[4 * b + 2] != kSelect) return;
  const int64_t vn = row_valid(valid_n, b, N);
  const float* row = scores + (size_t)b * N;
  const uint2* crow = cand + (size_t)b * N;
  const uint32_t* counts = cand_count + (size_t)b * blocks_per_row;
  uint8_t* mrow = mask + (size_t)b * N;
  __shared__ uint32_t h[kSelBins];
  __shared__ uint32_t s_wtot[kFinThreads / 64];
  __shared__ uint32_t s_out[2];
  __shared__ uint32_t s_off[kFinThreads];
  __shared__ uint2 s_cand[kFinLds];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // Candidate total, and the region offsets when a row has at most
  // kFinThreads slices (N <= 2^22).
  const bool small_rows = blocks_per_row <= kFinThreads;
  uint32_t C = 0;
  if (small_rows) {
    const int r = threadIdx.x;
    const uint32_t v = r < blocks_per_row ? counts[r] : 0u;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t u = __shfl_up(incl, off, 64);
      if (lane >= off) incl += u;
    }
    if (lane == 63) s_wtot[wave] = incl;
    __syncthreads();
    uint32_t below = 0;
    for (int w = 0; w < kFinThreads / 64; ++w) {
      below += w < wave ? s_wtot[w] : 0u;
      C += s_wtot[w];
    }
    if (r < blocks_per_row) s_off[r] = below + incl - v;
  } else {
    uint32_t part = 0;
    for (int r = threadIdx.x; r < blocks_per_row; r += kFinThreads) part += counts[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) s_wtot[wave] = part;
    __syncthreads();
    for (int w = 0; w < kFinThreads / 64; ++w) C += s_wtot[w];
  }
  __syncthreads();

  const uint32_t k = (uint32_t)top_k;
  uint32_t T, last;
  if (C >= k && small_rows && C <= (uint32_t)kFinLds) {
    // Stage the candidates; every pass then runs on LDS.
    for (int r = wave; r < blocks_per_row; r += kFinThreads / 64) {
      const uint32_t off = s_off[r];
      const uint32_t n_r = counts[r];
      for (uint32_t i = lane; i < n_r; i += 64) s_cand[off + i] = crow[(size_t)r * kSelSlice + i];
    }
    __syncthreads();
    auto each = [&](auto f) {
      for (uint32_t c = threadIdx.x; c < C; c += kFinThreads) f(s_cand[c]);
    };
    radix_select<kFinThreads>(each, k, h, s_wtot, s_out, &T, &last);
    each([&](uint2 e) {
      if (e.x > T || (e.x == T && e.y <= last)) mrow[e.y] = 1;
    });
  } else if (C >= k) {
    // Many candidates: read them from their regions in every pass.
    auto each = [&](auto f) {
      for (int r = wave; r < blocks_per_row; r += kFinThreads / 64) {
        const uint32_t n_r = counts[r];
        for (uint32_t i = lane; i < n_r; i += 64) f(crow[(size_t)r * kSelSlice + i]);
      }
    };
    radix_select<kFinThreads>(each, k, h, s_wtot, s_out, &T, &last);
    each([&](uint2 e) {
      if (e.x > T || (e.x == T && e.y <= last)) mrow[e.y] = 1;
    });
  } else {
    // Fewer than K keys reached the cut-off: select over the whole row.
    auto each = [&](auto f) {
      for (int64_t n = threadIdx.x; n < vn; n += kFinThreads) f(make_uint2(order_key(row[n]), (uint32_t)n));
    };
    radix_select<kFinThreads>(each, k, h, s_wtot, s_out, &T, &last);
    each([&](uint2 e) {
      if (e.x > T || (e.x == T && e.y <= last)) mrow[e.y] = 1;
    });
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
  hipLaunchKernelGGL(sel_sample_kernel, dim3(B), dim3(kSampleThreads), 0, stream, scores, N, valid_n, top_k,
                     ws.sel_state);
  hipLaunchKernelGGL(sel_collect_kernel, dim3(blocks_per_row, B), dim3(kSelThreads), 0, stream, scores, N, valid_n,
                     (const uint32_t*)ws.sel_state, (uint2*)ws.sel_cand, ws.sel_count, mask);
  hipLaunchKernelGGL(sel_final_kernel, dim3(B), dim3(kFinThreads), 0, stream, scores, N, valid_n, blocks_per_row,
                     top_k, (const uint32_t*)ws.sel_state, (const uint2*)ws.sel_cand, (const uint32_t*)ws.sel_count,
                     mask);
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
