// Attention-logit masking over a retrieval cycle (FlashMemory DS-V4
// Retriever README, "Inference flow": for the 64 decode steps after a
// retrieval cycle the attention logits of the chunks not kept are set to
// -inf; "What this simulates": a masked chunk contributes nothing to
// attention, as if its KV had not been loaded).
//
// logits [B][R][N] (R logit rows per request row: heads, query positions)
// are changed in place: -inf where mask[b][n] == 0, untouched elsewhere.
// grid = (ceil(N / 4096), B), 256 threads; thread t covers 16 consecutive
// chunks of its slice for every one of the row's R logit rows.  Per group of
// 16 chunks: all kept -> nothing; none kept -> one vector store of -inf (no
// read); mixed -> load, select, store.  Unaligned rows and the row tail use
// element stores.
#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kMaskThreads = 256;
constexpr int kMaskPer = 16;
constexpr int kMaskSlice = kMaskThreads * kMaskPer;

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

__device__ __forceinline__ uint32_t kept_bits16(const uint8_t* m, int bytes) {
  if (bytes == kMaskPer && (((uintptr_t)m) & 15) == 0) {
    const uint4 w = *(const uint4*)m;
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
    uint32_t bits = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t hi = (((a[q] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | a[q]) & 0x80808080u;  // byte != 0
      bits |= ((hi >> 7) & 1u) << (4 * q);
      bits |= ((hi >> 15) & 1u) << (4 * q + 1);
      bits |= ((hi >> 23) & 1u) << (4 * q + 2);
      bits |= ((hi >> 31) & 1u) << (4 * q + 3);
    }
    return bits;
  }
  uint32_t bits = 0;
  for (int j = 0; j < bytes; ++j) bits |= (m[j] != 0 ? 1u : 0u) << j;
  return bits;
}

template <typename E>
__global__ __launch_bounds__(kMaskThreads) void mask_logits_kernel(E* __restrict__ logits, int R, int64_t N,
                                                                   const uint8_t* __restrict__ mask) {
  typedef typename Elem<E>::Bits Bits;
  constexpr int kVec = 16 / sizeof(E);  // elements per 16-byte vector
  const int b = blockIdx.y;
  const int64_t n0 = (int64_t)blockIdx.x * kMaskSlice + (int64_t)threadIdx.x * kMaskPer;
  if (n0 >= N) return;
  const int cnt = N - n0 >= kMaskPer ? kMaskPer : (int)(N - n0);
  const uint32_t kept = kept_bits16(mask + (size_t)b * N + n0, cnt);
  const uint32_t all = (1u << cnt) - 1u;
  if (kept == all) return;  // nothing to mask in any of the R rows
  const Bits ninf = (Bits)Elem<E>::kNegInf;
  for (int r = 0; r < R; ++r) {
    Bits* p = (Bits*)(logits + ((size_t)b * R + r) * (size_t)N + n0);
    if (cnt == kMaskPer && (((uintptr_t)p) & 15) == 0) {
      uint4 v[kMaskPer / kVec];
      if (kept != 0) {
#pragma unroll
        for (int q = 0; q < kMaskPer / kVec; ++q) v[q] = ((const uint4*)p)[q];
      }
#pragma unroll
      for (int q = 0; q < kMaskPer / kVec; ++q) {
        Bits* e = (Bits*)&v[q];
#pragma unroll
        for (int i = 0; i < kVec; ++i)
          if (!((kept >> (q * kVec + i)) & 1u)) e[i] = ninf;
        ((uint4*)p)[q] = v[q];
      }
    } else {
      for (int j = 0; j < cnt; ++j)
        if (!((kept >> j) & 1u)) p[j] = ninf;
    }
  }
}

}  // namespace

hipError_t launch_mask_logits(void* logits, int dtype, int B, int R, int64_t N, const uint8_t* mask,
                              hipStream_t stream) {
  const dim3 grid((unsigned)((N + kMaskSlice - 1) / kMaskSlice), (unsigned)B);
  if (dtype == FM_DTYPE_BF16)
    hipLaunchKernelGGL(mask_logits_kernel<uint16_t>, grid, dim3(kMaskThreads), 0, stream, (uint16_t*)logits, R, N,
                       mask);
  else
    hipLaunchKernelGGL(mask_logits_kernel<float>, grid, dim3(kMaskThreads), 0, stream, (float*)logits, R, N, mask);
  return hipGetLastError();
}

}  // namespace fm
