// Resident set and recall delta of a retrieval cycle (FlashMemory-DeepSeek-V4
// model card, "How it works": every 64 decode steps the Memory Indexer's
// selection becomes the resident_set of chunks recalled from CPU to GPU;
// README "Inference flow": the keep mask of a cycle holds for the next 64
// steps).
//
// From this cycle's keep mask and the previous cycle's, per row:
//   resident = { n : mask[n] }                    (ascending)
//   entering = { n : mask[n] and not prev[n] }    (to recall)
//   leaving  = { n : prev[n] and not mask[n] }    (to evict)
// A mask byte counts as set when it is non-zero.
//
// Two passes over slices of kResSlice chunks (grid = slices x rows):
//   1. count: each block counts its slice's three sets, and each thread
//      keeps its 16 chunks' membership bits (one 8-byte word);
//   2. write: each block adds the counts of the slices before it (the list
//      offsets), scans its threads' counts, and writes its indices in order
//      from the kept bits (the masks are read once); the first slice's block
//      also writes the row totals.
// Every list is ascending because slices, threads and bytes are visited in
// index order.  Lists are capped at `cap` entries per row (the counts are
// the full sizes).
#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kResThreads = 256;
constexpr int kResPer = 16;  // chunks per thread: one 16-byte load per mask

__device__ __forceinline__ uint32_t wave_prefix_sum_u32(uint32_t v) {
  // Wave64 inclusive scan on DPP moves (row shifts, then row broadcasts).
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
  return v;
}

// Bit j of the result = byte j of the 16 bytes is non-zero.
__device__ __forceinline__ uint32_t nonzero_bits(uint4 w) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // High bit of each byte: set iff the byte is non-zero.
    const uint32_t hi = (((a[q] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | a[q]) & 0x80808080u;
    bits |= ((hi >> 7) & 1u) << (4 * q);
    bits |= ((hi >> 15) & 1u) << (4 * q + 1);
    bits |= ((hi >> 23) & 1u) << (4 * q + 2);
    bits |= ((hi >> 31) & 1u) << (4 * q + 3);
  }
  return bits;
}

struct SliceBits {
  uint32_t cur, enter, leave;  // bit j: chunk n0 + j is in the set
};

// Set bits of the 16 mask bytes at p (the first `bytes` of them; the rest
// count as 0): one 16-byte load when all 16 are in the row and 4-byte
// aligned, else byte loads.
__device__ __forceinline__ uint32_t mask_bits(const uint8_t* p, int bytes) {
  if (bytes == kResPer && (((uintptr_t)p) & 3) == 0) return nonzero_bits(*(const uint4*)p);
  uint32_t bits = 0;
  for (int j = 0; j < bytes; ++j) bits |= (p[j] != 0 ? 1u : 0u) << j;
  return bits;
}

// This thread's 16 chunks [n0, n0 + 16) of row b; chunks past N are unset.
__device__ __forceinline__ SliceBits load_bits(const uint8_t* prev, const uint8_t* mask, int b, int64_t N,
                                               int64_t n0) {
  const size_t off = (size_t)b * N + n0;
  const int bytes = N - n0 >= kResPer ? kResPer : (N > n0 ? (int)(N - n0) : 0);
  const uint32_t cur = mask_bits(mask + off, bytes);
  const uint32_t pv = prev ? mask_bits(prev + off, bytes) : 0u;
  return SliceBits{cur, cur & ~pv, pv & ~cur};
}

// Block sums of three counts (thread 0 gets them).
__device__ __forceinline__ uint3 block_sum3(uint3 v, uint32_t* s_w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v.x = __builtin_amdgcn_readlane(wave_prefix_sum_u32(v.x), 63);
  v.y = __builtin_amdgcn_readlane(wave_prefix_sum_u32(v.y), 63);
  v.z = __builtin_amdgcn_readlane(wave_prefix_sum_u32(v.z), 63);
  if (lane == 0) {
    s_w[3 * wave] = v.x;
    s_w[3 * wave + 1] = v.y;
    s_w[3 * wave + 2] = v.z;
  }
  __syncthreads();
  uint3 t = make_uint3(0, 0, 0);
#pragma unroll
  for (int w = 0; w < kResThreads / 64; ++w) {
    t.x += s_w[3 * w];
    t.y += s_w[3 * w + 1];
    t.z += s_w[3 * w + 2];
  }
  return t;
}

__global__ __launch_bounds__(kResThreads) void res_count_kernel(const uint8_t* prev, const uint8_t* mask, int64_t N,
                                                                uint32_t* counts, unsigned long long* bits) {
  __shared__ uint32_t s_w[3 * (kResThreads / 64)];
  const int b = blockIdx.y;
  const int64_t n0 = (int64_t)blockIdx.x * kResSlice + (int64_t)threadIdx.x * kResPer;
  const SliceBits sb = load_bits(prev, mask, b, N, n0);
  bits[((size_t)b * gridDim.x + blockIdx.x) * kResThreads + threadIdx.x] =
      (unsigned long long)sb.cur | ((unsigned long long)sb.enter << 16) | ((unsigned long long)sb.leave << 32);
  const uint3 t = block_sum3(make_uint3(__popc(sb.cur), __popc(sb.enter), __popc(sb.leave)), s_w);
  if (threadIdx.x == 0) {
    uint32_t* c = counts + ((size_t)b * gridDim.x + blockIdx.x) * 3;
    c[0] = t.x;
    c[1] = t.y;
    c[2] = t.z;
  }
}

__device__ __forceinline__ void write_list(uint32_t bits, int64_t n0, uint32_t pos, int32_t cap, int32_t* out) {
  while (bits) {
    const int j = __builtin_ctz(bits);
    bits &= bits - 1;
    if (pos < (uint32_t)cap) out[pos] = (int32_t)(n0 + j);
    ++pos;
  }
}

__global__ __launch_bounds__(kResThreads) void res_write_kernel(const unsigned long long* bits,
                                                                const uint32_t* counts, int32_t cap, int32_t* resident,
                                                                int32_t* n_resident, int32_t* entering,
                                                                int32_t* n_entering, int32_t* leaving,
                                                                int32_t* n_leaving) {
  __shared__ uint32_t s_w[3 * (kResThreads / 64)];
  const int b = blockIdx.y;
  const int slice = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)slice * kResSlice + (int64_t)threadIdx.x * kResPer;
  const unsigned long long kept = bits[((size_t)b * gridDim.x + slice) * kResThreads + threadIdx.x];
  const SliceBits sb{(uint32_t)kept & 0xffffu, (uint32_t)(kept >> 16) & 0xffffu, (uint32_t)(kept >> 32) & 0xffffu};

  // List offsets of this slice: the counts of the slices before it (and,
  // for slice 0, the row totals over all slices).
  const uint32_t* rc = counts + (size_t)b * gridDim.x * 3;
  const int upto = slice == 0 ? (int)gridDim.x : slice;
  uint3 part = make_uint3(0, 0, 0);
  for (int s = threadIdx.x; s < upto; s += kResThreads) {
    part.x += rc[3 * s];
    part.y += rc[3 * s + 1];
    part.z += rc[3 * s + 2];
  }
  const uint3 base_or_total = block_sum3(part, s_w);
  __syncthreads();  // s_w is reused below
  const uint3 base = slice == 0 ? make_uint3(0, 0, 0) : base_or_total;
  if (slice == 0 && threadIdx.x == 0) {
    n_resident[b] = (int32_t)base_or_total.x;
    if (n_entering) n_entering[b] = (int32_t)base_or_total.y;
    if (n_leaving) n_leaving[b] = (int32_t)base_or_total.z;
  }

  // Each thread's position within the slice: an exclusive block scan.
  const uint32_t c0 = __popc(sb.cur), c1 = __popc(sb.enter), c2 = __popc(sb.leave);
  const uint32_t i0 = wave_prefix_sum_u32(c0), i1 = wave_prefix_sum_u32(c1), i2 = wave_prefix_sum_u32(c2);
  if (lane == 63) {
    s_w[3 * wave] = i0;
    s_w[3 * wave + 1] = i1;
    s_w[3 * wave + 2] = i2;
  }
  __syncthreads();
  uint32_t p0 = base.x + i0 - c0, p1 = base.y + i1 - c1, p2 = base.z + i2 - c2;
#pragma unroll
  for (int w = 0; w < kResThreads / 64; ++w)
    if (w < wave) {
      p0 += s_w[3 * w];
      p1 += s_w[3 * w + 1];
      p2 += s_w[3 * w + 2];
    }
  const size_t ro = (size_t)b * cap;
  write_list(sb.cur, n0, p0, cap, resident + ro);
  if (entering) write_list(sb.enter, n0, p1, cap, entering + ro);
  if (leaving) write_list(sb.leave, n0, p2, cap, leaving + ro);
}

}  // namespace

hipError_t launch_resident_delta(const Workspace& ws, const uint8_t* prev, const uint8_t* mask, int B, int64_t N,
                                 int32_t cap, int32_t* resident, int32_t* n_resident, int32_t* entering,
                                 int32_t* n_entering, int32_t* leaving, int32_t* n_leaving, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kResSlice - 1) / kResSlice), (unsigned)B);
  hipLaunchKernelGGL(res_count_kernel, grid, dim3(kResThreads), 0, stream, prev, mask, N, ws.res_count, ws.res_bits);
  hipLaunchKernelGGL(res_write_kernel, grid, dim3(kResThreads), 0, stream, (const unsigned long long*)ws.res_bits,
                     (const uint32_t*)ws.res_count, cap, resident, n_resident, entering, n_entering, leaving,
                     n_leaving);
  return hipGetLastError();
}

}  // namespace fm
