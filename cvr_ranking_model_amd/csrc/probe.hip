// Bandwidth probes: the read ceilings that the streaming kernels are measured against.
//
// Two plain read kernels with no arithmetic beyond an xor that keeps the loads alive:
//   stream_read_kernel  reads a contiguous buffer once (the access pattern of the cross-attention,
//                       which streams every encoded state once per layer);
//   row_read_kernel     reads whole rows of a table at given ids (the access pattern of the
//                       embedding gather: the CTR article, section 二, keeps the hot embedding rows in
//                       HBM and reads them directly from the kernel).
// Each block writes one 32-bit xor of what it read, so the compiler cannot drop a load.  Both
// load plainly or with the nontemporal hint (NT), which is the faster form for data that cannot
// stay cached (a streaming read of 4 GiB: about 6.3 TB/s plain, 7.0 with the hint) and the
// slower one for a table part of which the last-level cache holds.  They are measurement tools,
// not part of scoring.
#include "../../include/cvr.h"
#include "device_common.h"
#include "kernels.h"
#include "model.h"

namespace cvr {

constexpr int kProbeThreads = 256;
constexpr int kStreamUnroll = 8;   // 16-byte loads in flight per lane
constexpr int kRowUnroll = 8;      // rows in flight per lane group

__device__ __forceinline__ uint32_t fold(const u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__device__ __forceinline__ void block_xor_store(uint32_t x, uint32_t* sink) {
  __shared__ uint32_t part[kProbeThreads / 64];
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) y ^= part[w];
    sink[blockIdx.x] = y;
  }
}

// n16: number of 16-byte vectors.  Each lane takes kStreamUnroll vectors a block-width apart per
// step, so every load instruction of a wave covers 1 KiB of consecutive bytes.
template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads * kStreamUnroll;
  uint32_t x = 0;
  for (int64_t base = (int64_t)blockIdx.x * kProbeThreads * kStreamUnroll + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kProbeThreads;
      v[u] = u32x4{0, 0, 0, 0};
      if (i < n16) v[u] = NT ? __builtin_nontemporal_load(&src[i]) : src[i];
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x ^= fold(v[u]);
  }
  block_xor_store(x, sink);
}

// LPR lanes read one row of LPR * 16 bytes; a group keeps kRowUnroll rows in flight.  An id
// outside [0, n_rows) reads row 0 (the probe takes no error path).
template <int LPR, bool NT>
__global__ __launch_bounds__(kProbeThreads) void row_read_kernel(const u32x4* __restrict__ table, int64_t n_rows,
                                                                const int32_t* __restrict__ ids, int64_t n_ids,
                                                                uint32_t* __restrict__ sink) {
  constexpr int kGroups = kProbeThreads / LPR;
  const int lane = threadIdx.x % LPR;
  const int64_t group = (int64_t)blockIdx.x * kGroups + threadIdx.x / LPR;
  const int64_t stride = (int64_t)gridDim.x * kGroups * kRowUnroll;
  uint32_t x = 0;
  for (int64_t base = group * kRowUnroll; base < n_ids; base += stride) {
    int64_t row[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t i = base + u;
      const int64_t r = i < n_ids ? (int64_t)ids[i] : -1;
      row[u] = (r >= 0 && r < n_rows) ? r : (i < n_ids ? 0 : -1);
    }
    u32x4 v[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      v[u] = u32x4{0, 0, 0, 0};
      if (row[u] >= 0) v[u] = NT ? __builtin_nontemporal_load(&table[row[u] * LPR + lane]) : table[row[u] * LPR + lane];
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) x ^= fold(v[u]);
  }
  block_xor_store(x, sink);
}

}  // namespace cvr

extern "C" cvr_status cvr_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks,
                                            int32_t nontemporal, void* hip_stream) {
  if (!src || !sink) return cvr::fail(nullptr, CVR_ERR_ARG, "null pointer");
  if (((uintptr_t)src & 15) || bytes < 0 || (bytes & 15)) return cvr::fail(nullptr, CVR_ERR_ARG, "src must be 16-byte aligned, bytes a multiple of 16");
  if (blocks < 1 || blocks > (1 << 20)) return cvr::fail(nullptr, CVR_ERR_ARG, "blocks outside [1, 2^20]");
  if (nontemporal != 0 && nontemporal != 1) return cvr::fail(nullptr, CVR_ERR_ARG, "nontemporal must be 0 or 1");
  if (nontemporal)
    cvr::launch_k(cvr::stream_read_kernel<true>, dim3(blocks), dim3(cvr::kProbeThreads), 0, (hipStream_t)hip_stream,
                  (const u32x4*)src, bytes / 16, sink);
  else
    cvr::launch_k(cvr::stream_read_kernel<false>, dim3(blocks), dim3(cvr::kProbeThreads), 0, (hipStream_t)hip_stream,
                  (const u32x4*)src, bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CVR_OK : cvr::fail(nullptr, CVR_ERR_HIP, hipGetErrorString(e));
}

extern "C" cvr_status cvr_probe_row_read(const void* table, int64_t n_rows, int32_t row_bytes, const int32_t* ids,
                                         int64_t n_ids, uint32_t* sink, int32_t blocks, int32_t nontemporal,
                                         void* hip_stream) {
  if (!table || !ids || !sink) return cvr::fail(nullptr, CVR_ERR_ARG, "null pointer");
  if (((uintptr_t)table & 15) || n_rows < 1 || n_ids < 0) return cvr::fail(nullptr, CVR_ERR_ARG, "bad table or sizes");
  if (blocks < 1 || blocks > (1 << 20)) return cvr::fail(nullptr, CVR_ERR_ARG, "blocks outside [1, 2^20]");
  if (nontemporal != 0 && nontemporal != 1) return cvr::fail(nullptr, CVR_ERR_ARG, "nontemporal must be 0 or 1");
  const hipStream_t st = (hipStream_t)hip_stream;
  const dim3 grid(blocks), block(cvr::kProbeThreads);
  const u32x4* t = (const u32x4*)table;
  auto go = [&](auto k) { cvr::launch_k(k, grid, block, 0, st, t, n_rows, ids, n_ids, sink); };
  switch (row_bytes * 2 + nontemporal) {
    case 128: go(cvr::row_read_kernel<4, false>); break;
    case 129: go(cvr::row_read_kernel<4, true>); break;
    case 256: go(cvr::row_read_kernel<8, false>); break;
    case 257: go(cvr::row_read_kernel<8, true>); break;
    case 512: go(cvr::row_read_kernel<16, false>); break;
    case 513: go(cvr::row_read_kernel<16, true>); break;
    default: return cvr::fail(nullptr, CVR_ERR_ARG, "row_bytes must be 64, 128 or 256");
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CVR_OK : cvr::fail(nullptr, CVR_ERR_HIP, hipGetErrorString(e));
}
