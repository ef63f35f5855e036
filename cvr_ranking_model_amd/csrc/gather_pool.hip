// Multi-table embedding gather with mean pooling, clamp and low-precision cast (steps A1-A2 / B1).
//
// One launch covers every sparse feature of the batch.  Blocks are assigned to
// features in contiguous ranges; inside a block, a group of dim/4 lanes owns one
// bag and each lane owns four consecutive columns (one 16-byte load per row), so
// a 64-dim row is one 256-byte coalesced access and a wave serves 4 (dim 64) or
// 8 (dim 32) bags at once.  Up to kUnroll rows of a bag are loaded before any is
// added, so many row fetches are in flight, but the adds happen in bag order:
// acc = 0; acc += row_0; acc += row_1; ...; pooled = acc / len (one correctly
// rounded fp32 division), matching the mean pooling of the CVR article
// (section 3.1, item 2) on fp32 embeddings (CTR article, section 三) bit for bit.
// The pooled value is clamped to +-clamp (NaN passes) and rounded to nearest-even
// into fp16/bf16 (CTR article, section 三), then written at the feature's column
// of the request-side or item-side input matrix.  A table kept in host memory behind an
// HBM hot-row cache is read through the cache (see CACHED below).
#include "device_common.h"
#include "kernels.h"

namespace cvr {

constexpr int kGatherThreads = 256;
constexpr int kUnroll = 8;

// CACHED: some feature of the launch reads a table that sits behind an HBM hot-row cache
// (CTR article, section 二).  For such a feature each id is looked up in its set: the group's
// first `ways` lanes read the set's tags and a ballot finds the way.  A hit reads the row from
// the cache and stamps the way with the batch number; a miss reads it from the host table and
// offers the lookup's position to the set's admission slot (atomicMin: the earliest miss of
// the batch is admitted after the gather; the miss that finds the slot empty queues the set).
// Either way the same fp32 row is added, so the pooled value does not depend on the cache.
// Hits and misses are summed per block and added to the cache's counters.
template <typename T, bool CACHED>
__global__ __launch_bounds__(kGatherThreads) void gather_pool_kernel(const GatherParams p) {
  const int b = blockIdx.x;
  int fi = 0;
#pragma unroll 1
  for (int k = 1; k < p.nf; ++k)
    if (p.f[k].block_begin <= b) fi = k;
  const GatherFeature& F = p.f[fi];
  const int lpb = F.dim >> 2;                       // lanes per bag
  const int bags_per_block = kGatherThreads / lpb;
  const int local = (b - F.block_begin) * bags_per_block + (int)threadIdx.x / lpb;
  const int lane = (int)threadIdx.x % lpb;
  constexpr bool cached = CACHED;                   // a launch holds only cached or only plain features
  if (!cached && local >= F.nbags) return;          // cached blocks stay for the counter reduction

  GatherCache C{};
  int epoch = 0;
  int gl = 0;
  if constexpr (cached) {
    C = p.cache[F.cache];
    epoch = C.hdr->epoch;
    gl = ((int)threadIdx.x & 63) - lane;              // the group's first lane in its wave
  }
  uint32_t hits = 0, misses = 0;
  if (local < F.nbags) {
    const int64_t g = F.bag_base + local;
    int64_t lo = p.bag_offsets[g];
    int64_t hi = p.bag_offsets[g + 1];
    // Malformed offsets are reported by the expand step; here they only must not lead outside ids.
    lo = lo < 0 ? 0 : (lo > p.n_ids ? p.n_ids : lo);
    hi = hi < lo ? lo : (hi > p.n_ids ? p.n_ids : hi);

    const float* __restrict__ tab = F.table + lane * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    bool bad = false;
    if constexpr (!cached) {
#pragma unroll 1
      for (int64_t j = lo; j < hi; j += kUnroll) {
        float4 r[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          r[u] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (j + u < hi) {
            const int32_t id = p.ids[j + u];
            if (id >= 0 && (int64_t)id < F.rows)
              r[u] = *reinterpret_cast<const float4*>(tab + (int64_t)id * F.dim);
            else
              bad = true;
          }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (j + u < hi) {
            acc.x += r[u].x;
            acc.y += r[u].y;
            acc.z += r[u].z;
            acc.w += r[u].w;
          }
        }
      }
    } else {
      // Same adds in the same order; the chunk's ids, then its sets' tags, then its rows are
      // each loaded together so that every step has kUnroll loads in flight.  Cache
      // bookkeeping (lane 0: the way each hit stamps, or the set each miss offers its position
      // to) is written after the rows are added: a store among the loads would make every
      // later load wait for it.
#pragma unroll 1
      for (int64_t j = lo; j < hi; j += kUnroll) {
        int32_t idv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) idv[u] = j + u < hi ? p.ids[j + u] : -1;
        bool ok[kUnroll];
        uint32_t set[kUnroll];
        int32_t tag[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          ok[u] = idv[u] >= 0 && (int64_t)idv[u] < F.rows;
          bad |= j + u < hi && !ok[u];
          set[u] = ok[u] ? fmix32((uint32_t)idv[u]) % (uint32_t)C.sets : 0u;
          tag[u] = ok[u] && lane < C.ways ? C.tags[(int64_t)set[u] * C.ways + lane] : -1;
        }
        int32_t note[kUnroll];
        float4 r[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const uint64_t found = (__ballot(ok[u] && tag[u] == idv[u]) >> gl) & ((1ull << C.ways) - 1);
          const int64_t base = (int64_t)set[u] * C.ways;
          const float* src = tab + (int64_t)(ok[u] ? idv[u] : 0) * F.dim;
          note[u] = -1;
          if (found) {
            const int way = __builtin_ctzll(found);
            src = C.rows + (base + way) * F.dim + lane * 4;
            note[u] = (int32_t)(base + way);
          } else if (ok[u]) {
            note[u] = -2 - (int32_t)set[u];
          }
          r[u] = ok[u] ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (j + u < hi) {
            acc.x += r[u].x;
            acc.y += r[u].y;
            acc.z += r[u].z;
            acc.w += r[u].w;
          }
        }
        if (lane == 0) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            if (note[u] >= 0) {
              C.stamps[note[u]] = epoch;
              ++hits;
            } else if (note[u] != -1) {
              // the first miss of this set in the batch queues the set for admission
              const int32_t sm = -2 - note[u];
              if (atomicMin(&C.first[sm], (int32_t)(j + u)) == INT32_MAX) C.queue[atomicAdd(&C.hdr->queued, 1)] = sm;
              ++misses;
            }
          }
        }
      }
    }
    if (bad) raise_flag(p.flag, ERRF_ID_RANGE);
    const int64_t len = hi - lo;
    if (len > 0) {
      const float fl = (float)len;
      acc.x = acc.x / fl;
      acc.y = acc.y / fl;
      acc.z = acc.z / fl;
      acc.w = acc.w / fl;
    }
    if (F.dbg) *reinterpret_cast<float4*>(F.dbg + (int64_t)local * F.dim + lane * 4) = acc;
    typedef typename Lowp<T>::vec4 V4;
    V4 o;
    o[0] = Lowp<T>::from_f32(clamp_keep_nan(acc.x, p.clamp));
    o[1] = Lowp<T>::from_f32(clamp_keep_nan(acc.y, p.clamp));
    o[2] = Lowp<T>::from_f32(clamp_keep_nan(acc.z, p.clamp));
    o[3] = Lowp<T>::from_f32(clamp_keep_nan(acc.w, p.clamp));
    T* out = reinterpret_cast<T*>(F.out) + (int64_t)local * F.ldo + F.col + lane * 4;
    *reinterpret_cast<V4*>(out) = o;
  }
  if constexpr (cached) {
    // Block totals of the lookups' outcomes (only each group's lane 0 counted).
    __shared__ uint32_t red[2][kGatherThreads / 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      hits += __shfl_xor(hits, off);
      misses += __shfl_xor(misses, off);
    }
    if ((threadIdx.x & 63) == 0) {
      red[0][threadIdx.x >> 6] = hits;
      red[1][threadIdx.x >> 6] = misses;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t h = 0, m = 0;
      for (int w = 0; w < kGatherThreads / 64; ++w) {
        h += red[0][w];
        m += red[1][w];
      }
      const int slot = blockIdx.x % kCacheCounterSlots;
      if (h + m) atomicAdd(&C.hdr->counters[CACHE_LOOKUPS][slot], (unsigned long long)(h + m));
      if (h) atomicAdd(&C.hdr->counters[CACHE_HITS][slot], (unsigned long long)h);
      if (m) atomicAdd(&C.hdr->counters[CACHE_MISSES][slot], (unsigned long long)m);
    }
  }
}

// Features read through a cache and plain features go to separate launches of their own
// instantiation, so the plain path keeps its register budget and load schedule.
template <bool CACHED>
static hipError_t launch_subset(const GatherParams& all, hipStream_t st) {
  GatherParams p = all;
  p.nf = 0;
  int blocks = 0;
  for (int k = 0; k < all.nf; ++k) {
    if ((all.f[k].cache >= 0) != CACHED) continue;
    GatherFeature& F = p.f[p.nf++];
    F = all.f[k];
    F.block_begin = blocks;
    const int bags_per_block = kGatherThreads / (F.dim / 4);
    blocks += (F.nbags + bags_per_block - 1) / bags_per_block;
  }
  p.total_blocks = blocks;
  if (blocks == 0) return hipSuccess;
  if (p.lowp == 0)
    launch_k(gather_pool_kernel<f16, CACHED>, dim3(blocks), dim3(kGatherThreads), 0, st, p);
  else
    launch_k(gather_pool_kernel<bf16, CACHED>, dim3(blocks), dim3(kGatherThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gather_pool(GatherParams& p, hipStream_t st) {
  hipError_t e = launch_subset<false>(p, st);
  if (e != hipSuccess) return e;
  return launch_subset<true>(p, st);
}

}  // namespace cvr
