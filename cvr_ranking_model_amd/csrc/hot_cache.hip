// HBM hot-row cache over a host-resident table (CTR article, section 二: hot embeddings in
// GPU HBM in front of host DRAM, least-recently-used replacement, hit/miss monitoring).
//
// The cache is set-associative: row r belongs to set fmix32(r) mod sets and may sit in any of
// the set's ways.  Time is counted in batches.  The gather looks every id up (hits read HBM
// and stamp the way with the batch number; misses read the host table over the bus and
// record the earliest missed lookup per set), then cache_admit_kernel lets each set that
// missed admit that one row into its least recently used way (an empty way first, then the
// smallest stamp, ties to the lowest way), copying the row from the host table.  Admitting at
// most one row per set per batch bounds the bus traffic a batch causes and keeps a batch from
// evicting the rows it has just read; the result is deterministic and independent of thread
// order, so the directory can be checked exactly against a reference.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace cvr {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

CacheLayout cache_layout(int64_t sets, int32_t ways, int32_t dim) {
  CacheLayout l{};
  const size_t entries = (size_t)sets * ways;
  l.tags = align256(sizeof(CacheHeader));
  l.stamps = align256(l.tags + entries * 4);
  l.first = align256(l.stamps + entries * 4);
  l.queue = align256(l.first + (size_t)sets * 4);
  l.rows = align256(l.queue + (size_t)sets * 4);
  l.total = align256(l.rows + entries * dim * 4);
  return l;
}

__global__ __launch_bounds__(256) void cache_init_kernel(const GatherCache c) {
  const int64_t entries = (int64_t)c.sets * c.ways;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < entries; i += stride) {
    c.tags[i] = -1;
    c.stamps[i] = 0;
  }
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < c.sets; i += stride) c.first[i] = INT32_MAX;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < CACHE_NCOUNTERS * kCacheCounterSlots; i += blockDim.x)
      (&c.hdr->counters[0][0])[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    c.hdr->epoch = 0;
    c.hdr->queued = 0;
  }
}

hipError_t launch_cache_init(const GatherCache& c, hipStream_t st) {
  const int64_t entries = (int64_t)c.sets * c.ways;
  const int blocks = (int)std::min<int64_t>(4096, (entries + 255) / 256);
  launch_k(cache_init_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st, c);
  return hipGetLastError();
}

struct CacheBeginArgs {
  CacheHeader* hdr[kMaxCaches];
  int32_t n;
};

__global__ void cache_begin_kernel(const CacheBeginArgs a) {
  if ((int)threadIdx.x < a.n) {
    a.hdr[threadIdx.x]->epoch += 1;
    a.hdr[threadIdx.x]->queued = 0;
  }
}

hipError_t launch_cache_begin(CacheHeader* const* hdrs, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n > kMaxCaches) return hipErrorInvalidValue;
  CacheBeginArgs a{};
  for (int i = 0; i < n; ++i) a.hdr[i] = hdrs[i];
  a.n = n;
  launch_k(cache_begin_kernel, dim3(1), dim3(64), 0, st, a);
  return hipGetLastError();
}

// One group of dim/4 lanes per queued set (the gather queued each set that missed once):
// every lane reads the set's directory and picks the same victim way; each lane copies four
// floats of the admitted row; lane 0 updates the directory.  Groups stride over the queue.
__global__ __launch_bounds__(256) void cache_admit_kernel(const GatherCache c, const int32_t* __restrict__ ids,
                                                          int64_t n_ids, const float* __restrict__ host,
                                                          int64_t rows, int32_t dim) {
  const int lpb = dim >> 2;
  const int gpb = 256 / lpb;
  const int lane = (int)threadIdx.x % lpb;
  const int queued = min(c.hdr->queued, c.sets);
  uint32_t adm = 0, ev = 0;
#pragma unroll 1
  for (int q = blockIdx.x * gpb + (int)threadIdx.x / lpb; q < queued; q += gridDim.x * gpb) {
    const int64_t s = c.queue[q];
    if (s < 0 || s >= c.sets) continue;
    const int32_t j = c.first[s];
    // A position is only ever offered for an id inside the table; the checks keep a slot left
    // over from an interrupted call from reading outside the arrays.
    const int32_t row = j >= 0 && j < n_ids ? ids[j] : -1;
    if (row >= 0 && row < rows) {
      const int64_t base = s * c.ways;
      int victim = -1;
      for (int w = 0; w < c.ways; ++w)
        if (c.tags[base + w] < 0) {
          victim = w;
          break;
        }
      const bool evict = victim < 0;
      if (evict) {
        int best = INT32_MAX;
        for (int w = 0; w < c.ways; ++w) {
          const int32_t stamp = c.stamps[base + w];
          if (stamp < best) {
            best = stamp;
            victim = w;
          }
        }
      }
      const float4 v = *reinterpret_cast<const float4*>(host + (int64_t)row * dim + lane * 4);
      *reinterpret_cast<float4*>(c.rows + (base + victim) * dim + lane * 4) = v;
      if (lane == 0) {
        c.tags[base + victim] = row;
        c.stamps[base + victim] = c.hdr->epoch;
        adm += 1;
        ev += evict ? 1 : 0;
      }
    }
    if (j != INT32_MAX && lane == 0) c.first[s] = INT32_MAX;
  }
  __shared__ uint32_t red[2][4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    adm += __shfl_xor(adm, off);
    ev += __shfl_xor(ev, off);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = adm;
    red[1][threadIdx.x >> 6] = ev;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t a = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const uint32_t e = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    const int slot = blockIdx.x % kCacheCounterSlots;
    if (a) atomicAdd(&c.hdr->counters[CACHE_ADMISSIONS][slot], (unsigned long long)a);
    if (e) atomicAdd(&c.hdr->counters[CACHE_EVICTIONS][slot], (unsigned long long)e);
  }
}

hipError_t launch_cache_admit(const GatherCache& c, const int32_t* ids, int64_t n_ids, const float* host_table,
                              int64_t rows, int32_t dim, int64_t max_lookups, hipStream_t st) {
  if (dim < 4 || dim % 4 || dim > 256 || c.sets <= 0) return hipErrorInvalidValue;
  const int per_block = 256 / (dim / 4);
  const int64_t most = std::max<int64_t>(1, std::min<int64_t>(c.sets, max_lookups));
  const int64_t blocks = std::min<int64_t>(2048, (most + per_block - 1) / per_block);
  launch_k(cache_admit_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, ids, n_ids, host_table, rows, dim);
  return hipGetLastError();
}

}  // namespace cvr
