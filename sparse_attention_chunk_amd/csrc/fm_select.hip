// Keep masks (FlashMemory DS-V4 Retriever README, "Usage": select_topk with
// top_k=... or threshold=...; "Inference flow": keep_mask = top-K of the
// scores, or sigmoid > thresh).
//
// Top-K is an exact per-row selection on order-preserving 32-bit keys of the
// fp32 scores; ties at the K-th key go to the lowest chunk indices, which
// makes the mask unique.  Three kernels per call:
//   1. sample: one block per row reads 4096 keys (64 runs of 64 chunks
//      spread over the row; the whole row when it is shorter) and picks a
//      cut-off L, the m-th largest sampled key, with m chosen so that about
//      K plus four standard deviations of the row's keys are expected at or
//      above L (a row that fits in the sample gets its exact K-th key);
//   2. collect: one pass over the row writes the mask (0 everywhere, 1 for
//      every valid chunk when K keeps them all) and writes the (key, index)
//      pairs of keys >= L to the row's candidate list, one region per block;
//   3. final: one block per row selects exactly among the candidates: radix
//      passes over the key give the K-th largest key T and how many keys equal
//      to T are kept, radix passes over the index of the keys equal to T (only
//      when some are left out) give the last index kept; those candidates'
//      mask bytes are set.  When fewer
//      than K keys reached L (the sample was unrepresentative), the same
//      passes run over the whole row instead, so the result is always exact.
#include "fm_radix.h"

namespace fm {
namespace {

using namespace radix;

__device__ inline int64_t row_valid(const int32_t* valid_n, int b, int64_t N) {
  if (!valid_n) return N;
  const int64_t v = valid_n[b];
  return v < 0 ? 0 : (v > N ? N : v);
}

// state[b] = {cut-off L, unused, mode, unused}
enum : uint32_t { kSelect = 0, kKeepAll = 1, kKeepNone = 2 };

constexpr int kTile16 = 16;  // chunks per tile of the score pass (tile maxima)
constexpr int kSampleRuns = 64;
constexpr int kSampleRun = 64;
constexpr int kSampleSize = kSampleRuns * kSampleRun;  // 4096
constexpr int kSampleThreads = 1024;
constexpr int kSamplePerThread = kSampleSize / kSampleThreads;  // 4

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
  __shared__ __attribute__((aligned(16))) uint32_t h[2 * kSelBins];
  __shared__ uint32_t s_wtot[kSampleThreads / 64];
  __shared__ uint32_t s_out[3];
  const float* row = scores + (size_t)b * N;
  const bool whole = vn <= kSampleSize;
  const uint32_t S = whole ? (uint32_t)vn : (uint32_t)kSampleSize;
  // Sample i = t + kSampleThreads * j sits in run r = i / kSampleRun at
  // offset t % kSampleRun; run r starts at r (vn - kSampleRun) / 63 (32-bit:
  // 63 * 2^26 fits).  Loads go through a descriptor over the row's valid
  // scores with no branch, all issued before the first use.
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, (int)(vn * 4), 0x00020000);
  const uint32_t span = whole ? 0u : (uint32_t)(vn - kSampleRun);
  float v[kSamplePerThread];
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) {
    const uint32_t i = (uint32_t)t + kSampleThreads * j;
    const uint32_t r = i / kSampleRun;
    const uint32_t n = whole ? i : r * span / (kSampleRuns - 1) + (i % kSampleRun);
    v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, 4u * n, 0, 0));
  }
  uint32_t kr[kSamplePerThread];
#pragma unroll
  for (int j = 0; j < kSamplePerThread; ++j) kr[j] = order_key(v[j]);
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
#pragma unroll
        for (int j = 0; j < kSamplePerThread; ++j) {
          const uint32_t i = (uint32_t)t + kSampleThreads * j;
          if (i < S) f(make_uint2(kr[j], i));
        }
      },
      m, 0, h, s_wtot, s_out, &L, &unused);
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
  const uint32_t incl = wave_prefix_sum(mine);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
constexpr int kFinLds = 8192;  // candidates held in registers (8 per thread); more are read from their regions each pass

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
  __shared__ __attribute__((aligned(16))) uint32_t h[2 * kSelBins];
  __shared__ uint32_t s_wtot[kFinThreads / 64];
  __shared__ uint32_t s_out[3];
  __shared__ uint32_t s_off[kFinThreads];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // Candidate total, and the region offsets when a row has at most
  // kFinThreads slices (N <= 2^22).
  const bool small_rows = blocks_per_row <= kFinThreads;
  uint32_t C = 0;
  if (small_rows) {
    const int r = threadIdx.x;
    const uint32_t v = r < blocks_per_row ? counts[r] : 0u;
    const uint32_t incl = wave_prefix_sum(v);
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
    part = wave_sum_u32(part);
    if (lane == 0) s_wtot[wave] = part;
    __syncthreads();
    for (int w = 0; w < kFinThreads / 64; ++w) C += s_wtot[w];
  }
  __syncthreads();

  const uint32_t k = (uint32_t)top_k;
  const int ib = index_bits(vn);
  uint32_t T, last;
  if (C >= k && small_rows && C <= (uint32_t)kFinLds) {
    // The candidates stay in registers for every pass.  Candidate c lies in
    // the slice r with s_off[r] <= c < s_off[r + 1] (binary search); all of a
    // thread's loads are issued together.
    constexpr int kPer = kFinLds / kFinThreads;
    uint2 v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t c = threadIdx.x + kFinThreads * j;
      v[j] = make_uint2(0u, 0u);
      if (c < C) {
        int lo = 0, hi = blocks_per_row - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_off[mid] <= c) lo = mid;
          else hi = mid - 1;
        }
        v[j] = crow[(size_t)lo * kSelSlice + (c - s_off[lo])];
      }
    }
    auto each = [&](auto f) {
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (threadIdx.x + kFinThreads * j < C) f(v[j]);
    };
    radix_select<kFinThreads>(each, k, ib, h, s_wtot, s_out, &T, &last);
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
    radix_select<kFinThreads>(each, k, ib, h, s_wtot, s_out, &T, &last);
    each([&](uint2 e) {
      if (e.x > T || (e.x == T && e.y <= last)) mrow[e.y] = 1;
    });
  } else {
    // Fewer than K keys reached the cut-off: select over the whole row.
    auto each = [&](auto f) {
      for (int64_t n = threadIdx.x; n < vn; n += kFinThreads) f(make_uint2(order_key(row[n]), (uint32_t)n));
    };
    radix_select<kFinThreads>(each, k, ib, h, s_wtot, s_out, &T, &last);
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

// Top-K finished from the score pass's histograms and tile maxima (the
// selection folded into fm_score_topk).  grid = B, block = 1024.  Per row:
//   1. the row's histogram: the global one (rows a block reached past its
//      two slots) plus slot 0 of every block whose first row is this row and
//      slot 1 of every block whose first row is the one before;
//   2. the bin c holding the K-th largest score, the count A above it and
//      its own count n_c (K <= A + n_c);
//   3. the tiles whose largest score falls in bin c or above (at most
//      A + n_c of them);
//   4. their chunks: above bin c the mask byte is set (every such chunk is
//      among the top K), in bin c the (key, index) pair becomes a candidate;
//   5. the K - A candidates kept: all of them, or an exact radix selection
//      (key descending, index ascending).
// When the tiles or the candidates overflow LDS (many equal or nearly equal
// scores), the row is selected exactly from all its scores instead.  The
// result is the mask fm_select_topk gives for the same scores.
constexpr int kFinishThreads = 1024;
constexpr int kFinishTiles = 2048;      // qualifying tiles held in LDS
constexpr int kFinishCand = 4096;       // candidates of bin c held in LDS
constexpr int kFinishBatch = 16;        // loads issued together

__device__ __forceinline__ int fused_bin(float e) {
  const int b = (int)(e * (float)kHistBins);
  return b < kHistBins - 1 ? b : kHistBins - 1;
}

__global__ __launch_bounds__(kFinishThreads) void topk_finish_kernel(
    const float* __restrict__ scores, int64_t N, const int32_t* __restrict__ valid_n, int32_t top_k,
    const uint32_t* __restrict__ sel_hist, const int32_t* __restrict__ block_row0, int nblocks,
    const uint32_t* __restrict__ hist_x, const float* __restrict__ tile_max, uint8_t* __restrict__ mask) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int64_t vn = row_valid(valid_n, b, N);
  uint8_t* mrow = mask + (size_t)b * N;
  const float* row = scores + (size_t)b * N;
  if (top_k == 0 || vn == 0) return;  // the score pass wrote zeros
  if ((int64_t)top_k >= vn) {
    for (int64_t n = t; n < vn; n += kFinishThreads) mrow[n] = 1;
    return;
  }
  __shared__ __attribute__((aligned(16))) uint32_t h[2 * kSelBins];
  __shared__ uint32_t s_q[kFinishTiles];
  __shared__ uint2 s_c[kFinishCand];
  __shared__ uint32_t s_wtot[kFinishThreads / 64];
  __shared__ uint32_t s_out[3];
  __shared__ unsigned long long s_bm[2][kFinishThreads / 64];
  __shared__ uint32_t s_blk[kMaxScoreBlocks];  // a block matches at most one of the two slots
  __shared__ uint32_t s_nblk, s_nq, s_nc;

  // 1. Histogram slots of this row.
  {
    bool h0 = false, h1 = false;
    if (t < nblocks) {
      const int r0 = block_row0[t];
      h0 = r0 == b;
      h1 = r0 >= 0 && r0 == b - 1;
    }
    const unsigned long long m0 = __ballot(h0), m1 = __ballot(h1);
    if (lane == 0) {
      s_bm[0][wave] = m0;
      s_bm[1][wave] = m1;
    }
    __syncthreads();
    if (t == 0) {
      uint32_t n = 0;
      for (int slot = 0; slot < 2; ++slot)
        for (int w = 0; w < kFinishThreads / 64; ++w)
          for (unsigned long long m = s_bm[slot][w]; m; m &= m - 1)
            s_blk[n++] = (uint32_t)(2 * (w * 64 + __builtin_ctzll(m)) + slot);
      s_nblk = n;
      s_nq = 0;
      s_nc = 0;
    }
    __syncthreads();
    uint2 c = *(const uint2*)(hist_x + (size_t)b * kHistBins + 2 * t);
    const uint32_t nblk = s_nblk;
    for (uint32_t base = 0; base < nblk; base += kFinishBatch) {
      uint2 x[kFinishBatch];
#pragma unroll
      for (int j = 0; j < kFinishBatch; ++j)
        x[j] = base + j < nblk ? *(const uint2*)(sel_hist + (size_t)s_blk[base + j] * kHistBins + 2 * t)
                               : make_uint2(0u, 0u);
#pragma unroll
      for (int j = 0; j < kFinishBatch; ++j) {
        c.x += x[j].x;
        c.y += x[j].y;
      }
    }
    *(uint2*)(h + 2 * t) = c;
  }
  __syncthreads();
  // 2. The cut-off bin.
  block_find<kFinishThreads>(h, (uint32_t)top_k, s_wtot, s_out, true);
  const int cbin = (int)s_out[0];
  const uint32_t above = s_out[1], n_c = s_out[2];
  const uint32_t need = (uint32_t)top_k - above;
  bool exact_row = n_c > (uint32_t)kFinishCand;
  if (!exact_row) {
    // 3. Qualifying tiles.
    const int64_t nt = (vn + kTile16 - 1) / kTile16;
    const float* trow = tile_max + (size_t)b * ((N + kTile16 - 1) / kTile16);
    for (int64_t base = t; base < nt; base += (int64_t)kFinishThreads * kFinishBatch) {
      float m[kFinishBatch];
#pragma unroll
      for (int j = 0; j < kFinishBatch; ++j) {
        const int64_t i = base + (int64_t)j * kFinishThreads;
        m[j] = i < nt ? trow[i] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kFinishBatch; ++j) {
        const int64_t i = base + (int64_t)j * kFinishThreads;
        if (i < nt && fused_bin(m[j]) >= cbin) {
          const uint32_t pos = atomicAdd(&s_nq, 1u);
          if (pos < (uint32_t)kFinishTiles) s_q[pos] = (uint32_t)i;
        }
      }
    }
    __syncthreads();
    const uint32_t nq = s_nq;
    exact_row = nq > (uint32_t)kFinishTiles;
    if (!exact_row) {
      // 4. Their chunks.
      const uint32_t total = nq * kTile16;
      for (uint32_t base = t; base < total; base += kFinishThreads * kFinishBatch) {
        float e[kFinishBatch];
        int64_t n[kFinishBatch];
#pragma unroll
        for (int j = 0; j < kFinishBatch; ++j) {
          const uint32_t x = base + j * kFinishThreads;
          n[j] = x < total ? (int64_t)s_q[x / kTile16] * kTile16 + (x % kTile16) : vn;
          e[j] = n[j] < vn ? row[n[j]] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kFinishBatch; ++j) {
          if (n[j] < vn) {
            const int bn = fused_bin(e[j]);
            if (bn > cbin) {
              mrow[n[j]] = 1;
            } else if (bn == cbin) {
              const uint32_t pos = atomicAdd(&s_nc, 1u);
              if (pos < (uint32_t)kFinishCand) s_c[pos] = make_uint2(order_key(e[j]), (uint32_t)n[j]);
            }
          }
        }
      }
      __syncthreads();
      // 5. The K - A kept of bin c.
      const uint32_t nc = s_nc < (uint32_t)kFinishCand ? s_nc : (uint32_t)kFinishCand;
      if (need >= nc) {
        for (uint32_t i = t; i < nc; i += kFinishThreads) mrow[s_c[i].y] = 1;
      } else {
        auto each = [&](auto f) {
          for (uint32_t i = t; i < nc; i += kFinishThreads) f(s_c[i]);
        };
        uint32_t T, last;
        radix_select<kFinishThreads>(each, need, index_bits(vn), h, s_wtot, s_out, &T, &last);
        each([&](uint2 e) {
          if (e.x > T || (e.x == T && e.y <= last)) mrow[e.y] = 1;
        });
      }
      return;
    }
  }
  // Too many equal or nearly equal scores for LDS: exact selection over the
  // whole row (the mask bytes set in step 4 are all among the top K).
  auto each = [&](auto f) {
    for (int64_t n = t; n < vn; n += kFinishThreads) f(make_uint2(order_key(row[n]), (uint32_t)n));
  };
  uint32_t T, last;
  radix_select<kFinishThreads>(each, (uint32_t)top_k, index_bits(vn), h, s_wtot, s_out, &T, &last);
  each([&](uint2 e) {
    if (e.x > T || (e.x == T && e.y <= last)) mrow[e.y] = 1;
  });
}

}  // namespace

hipError_t launch_topk_finish(const Workspace& ws, const float* scores, int B, int64_t N, const int32_t* valid_n,
                              int32_t top_k, uint8_t* mask, hipStream_t stream) {
  hipLaunchKernelGGL(topk_finish_kernel, dim3(B), dim3(kFinishThreads), 0, stream, scores, N, valid_n, top_k,
                     (const uint32_t*)ws.sel_hist, (const int32_t*)ws.block_row0, ws.score_blocks,
                     (const uint32_t*)ws.sel_hist_x, (const float*)ws.tile_max, mask);
  return hipGetLastError();
}

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
