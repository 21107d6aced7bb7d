// Attention-logit masking over a retrieval cycle (FlashMemory DS-V4
// Retriever README, "Inference flow": for the 64 decode steps after a
// retrieval cycle the attention logits of the chunks not kept are set to
// -inf; "What this simulates": a masked chunk contributes nothing to
// attention, as if its KV had not been loaded).
//
// logits [B][R][N] (R logit rows per request row: heads, query positions)
// are changed in place: -inf where mask[b][n] == 0, untouched elsewhere.
// Stores are the cost.  A block takes one segment of kMaskVecs x 256
// 16-byte vectors of a request row's chunks and kMaskRows of its logit rows;
// instruction i of thread t handles vector i * 256 + t, so every store
// instruction of a block covers 4 KB.  The mask bits of the segment are read
// once per block, and they are the same for all of the block's logit rows.
// Per vector: all kept -> nothing; none kept -> a store of -inf, no read;
// mixed -> load, select, store.  The loads of a thread's first mixed vector
// are issued for every row of the block before the -inf stores, so their
// latency hides behind the stores.  With 0.2% of the chunks kept, 12% of the
// 128-byte lines hold a kept element, and those lines are read as well as
// written.  Every store is non-temporal: with ordinary stores the reads of
// the mixed lines slowed the whole write stream (B=30, 64 bf16 logit rows,
// N=262144: 272 us with a top-512 mask against 192 us with nothing kept);
// non-temporal, with one vector per thread and four rows per block, 159 us
// and 166 us (a plain fill of the same bytes: 146 us).  Rows whose length is
// not a whole number of vectors use element stores.
#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kMaskThreads = 256;
constexpr int kMaskVecs = 1;   // 16-byte vectors per thread per logit row
constexpr int kMaskRows = 4;   // logit rows per block

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_nt(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4*)p);
}

template <typename E>
struct Elem;
template <>
struct Elem<float> {
  static constexpr uint32_t kNegInf = 0xff800000u;
  typedef uint32_t Bits;
};
template <>
struct Elem<uint16_t> {  // bf16
  static constexpr uint32_t kNegInf = 0xff80u;
  typedef uint16_t Bits;
};

// Bit j: mask byte j of the V bytes at m is non-zero.
template <int V>
__device__ __forceinline__ uint32_t kept_bits(const uint8_t* m) {
  uint32_t w[2];
  if constexpr (V == 8) {
    const uint2 x = *(const uint2*)m;
    w[0] = x.x;
    w[1] = x.y;
  } else {
    w[0] = *(const uint32_t*)m;
    w[1] = 0;
  }
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < V / 4; ++q) {
    const uint32_t hi = (((w[q] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w[q]) & 0x80808080u;  // byte != 0
    bits |= ((hi >> 7) & 1u) << (4 * q);
    bits |= ((hi >> 15) & 1u) << (4 * q + 1);
    bits |= ((hi >> 23) & 1u) << (4 * q + 2);
    bits |= ((hi >> 31) & 1u) << (4 * q + 3);
  }
  return bits;
}

// grid = (segments, row groups of kMaskRows, B).  VEC: every row holds a
// whole number of vectors and the buffers are aligned (N % V == 0).
template <typename E, bool VEC>
__global__ __launch_bounds__(kMaskThreads) void mask_logits_kernel(E* __restrict__ logits, int R, int64_t N,
                                                                   const uint8_t* __restrict__ mask) {
  typedef typename Elem<E>::Bits Bits;
  constexpr int V = 16 / sizeof(E);  // elements per vector
  constexpr int64_t kSeg = (int64_t)kMaskThreads * kMaskVecs * V;
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * kMaskRows;
  const int r1 = r0 + kMaskRows < R ? r0 + kMaskRows : R;
  const int64_t e0 = (int64_t)blockIdx.x * kSeg;
  const uint8_t* mrow = mask + (size_t)b * N;
  const Bits ninf = (Bits)Elem<E>::kNegInf;
  if constexpr (VEC) {
    const uint32_t all = (1u << V) - 1u;
    uint64_t kb = 0;                // V kept bits per vector
    uint32_t none = 0, mixed = 0;   // bit i: vector i has no kept element / some but not all
#pragma unroll
    for (int i = 0; i < kMaskVecs; ++i) {
      const int64_t e = e0 + ((int64_t)i * kMaskThreads + threadIdx.x) * V;
      const uint32_t k = e < N ? kept_bits<V>(mrow + e) : all;  // past the row: nothing to do
      kb |= (uint64_t)k << (V * i);
      none |= (k == 0 ? 1u : 0u) << i;
      mixed |= (k != 0 && k != all ? 1u : 0u) << i;
    }
    const uint32_t w = sizeof(Bits) == 2 ? (Elem<E>::kNegInf | (Elem<E>::kNegInf << 16)) : Elem<E>::kNegInf;
    const uint4 fill = make_uint4(w, w, w, w);
    uint4* base = (uint4*)(logits + (size_t)b * R * (size_t)N + e0) + threadIdx.x;
    const size_t rstride = (size_t)N / V;  // vectors per logit row
    auto at = [&](int r, int i) { return base + (size_t)r * rstride + (size_t)i * kMaskThreads; };
    uint4 v[kMaskRows];
    if (mixed) {
      const int i = __builtin_ctz(mixed);
#pragma unroll
      for (int rr = 0; rr < kMaskRows; ++rr)
        if (r0 + rr < r1) v[rr] = *at(r0 + rr, i);
    }
    for (int r = r0; r < r1; ++r) {
#pragma unroll
      for (int i = 0; i < kMaskVecs; ++i)
        if ((none >> i) & 1u) store_nt(at(r, i), fill);
    }
    for (bool first = true; mixed; first = false) {
      const int i = __builtin_ctz(mixed);
      mixed &= mixed - 1;
      const uint32_t k = (uint32_t)(kb >> (V * i)) & all;
      if (!first) {
#pragma unroll
        for (int rr = 0; rr < kMaskRows; ++rr)
          if (r0 + rr < r1) v[rr] = *at(r0 + rr, i);
      }
#pragma unroll
      for (int rr = 0; rr < kMaskRows; ++rr) {
        if (r0 + rr >= r1) continue;
        Bits* el = (Bits*)&v[rr];
#pragma unroll
        for (int j = 0; j < V; ++j)
          if (!((k >> j) & 1u)) el[j] = ninf;
        store_nt(at(r0 + rr, i), v[rr]);
      }
    }
  } else {
    for (int r = r0; r < r1; ++r) {
      Bits* p = (Bits*)(logits + ((size_t)b * R + r) * (size_t)N);
      for (int64_t e = e0 + threadIdx.x; e < e0 + kSeg && e < N; e += kMaskThreads)
        if (mrow[e] == 0) p[e] = ninf;
    }
  }
}

}  // namespace

hipError_t launch_mask_logits(void* logits, int dtype, int B, int R, int64_t N, const uint8_t* mask,
                              hipStream_t stream) {
  const int V = dtype == FM_DTYPE_BF16 ? 8 : 4;
  const int64_t seg = (int64_t)kMaskThreads * kMaskVecs * V;
  const dim3 grid((unsigned)((N + seg - 1) / seg), (unsigned)((R + kMaskRows - 1) / kMaskRows), (unsigned)B);
  const bool vec = N % V == 0 && ((uintptr_t)logits & 15) == 0 && ((uintptr_t)mask & 7) == 0;
  if (dtype == FM_DTYPE_BF16) {
    if (vec)
      hipLaunchKernelGGL((mask_logits_kernel<uint16_t, true>), grid, dim3(kMaskThreads), 0, stream, (uint16_t*)logits,
                         R, N, mask);
    else
      hipLaunchKernelGGL((mask_logits_kernel<uint16_t, false>), grid, dim3(kMaskThreads), 0, stream,
                         (uint16_t*)logits, R, N, mask);
  } else {
    if (vec)
      hipLaunchKernelGGL((mask_logits_kernel<float, true>), grid, dim3(kMaskThreads), 0, stream, (float*)logits, R, N,
                         mask);
    else
      hipLaunchKernelGGL((mask_logits_kernel<float, false>), grid, dim3(kMaskThreads), 0, stream, (float*)logits, R,
                         N, mask);
  }
  return hipGetLastError();
}

}  // namespace fm
