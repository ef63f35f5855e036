// The sequence chunk plan (steps B3-B5): the exclusive scan of each (sequence, request)
// segment's chunk count and one descriptor per chunk, for the kernels of seq.hip.  Shared by the
// plan's own launch and the launch that also runs the batch expansion (expand.hip).
#ifndef CVR_CHUNK_PLAN_H
#define CVR_CHUNK_PLAN_H

#include "device_common.h"
#include "kernels.h"

namespace cvr {

// Positions of segment g = s * R + r, clamped to [0, n_positions] and non-decreasing.
__device__ __forceinline__ void segment_range(const int32_t* __restrict__ seq_offsets, int R, int g, int64_t n_positions,
                                              int64_t& a, int64_t& e) {
  const int s = g / R, r = g % R;
  a = seq_offsets[(int64_t)s * (R + 1) + r];
  e = seq_offsets[(int64_t)s * (R + 1) + r + 1];
  a = a < 0 ? 0 : (a > n_positions ? n_positions : a);
  e = e < a ? a : (e > n_positions ? n_positions : e);
}

// One block of 1024 threads of a plan launch of nb blocks: every block runs the scan of the
// segment lengths into LDS (`off`, S*R+1 entries; the offsets are few and sit in L2 after the
// first block reads them), block 0 writes the table out for the kernels that follow, and each
// block then writes the descriptors of its share of the chunks, searching the table in LDS.
// Offsets are 64-bit sums capped at max_chunks, so malformed offsets (flagged by the expand
// kernel) keep every chunk inside its own segment and the arrays.
__device__ __forceinline__ void chunk_plan_block(const PlanParams& q, int b, int nb, int32_t* __restrict__ off,
                                                 long long* __restrict__ wsum) {
  const int SR = q.S * q.R;
  const int per = (SR + 1023) / 1024;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g0 = t * per;
  long long local = 0;
  for (int g = g0; g < g0 + per && g < SR; ++g) {
    int64_t a, e;
    segment_range(q.seq_offsets, q.R, g, q.n_positions, a, e);
    local += (e - a + kSeqChunk - 1) / kSeqChunk;
  }
  long long incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    long long x = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const long long v = __shfl_up(x, o);
      if (lane >= o) x += v;
    }
    if (lane < 16) wsum[lane] = x;
  }
  __syncthreads();
  long long run = (w > 0 ? wsum[w - 1] : 0) + incl - local;
  for (int g = g0; g < g0 + per && g < SR; ++g) {
    off[g] = (int32_t)(run < q.max_chunks ? run : q.max_chunks);
    int64_t a, e;
    segment_range(q.seq_offsets, q.R, g, q.n_positions, a, e);
    run += (e - a + kSeqChunk - 1) / kSeqChunk;
  }
  if (t == 1023) off[SR] = (int32_t)(wsum[15] < q.max_chunks ? wsum[15] : q.max_chunks);
  __syncthreads();
  if (b == 0)
    for (int g = t; g <= SR; g += 1024) q.chunk_off[g] = off[g];
  const int total = off[SR];
  const int share = (total + nb - 1) / nb;
  const int c0 = b * share;
  const int c1 = c0 + share < total ? c0 + share : total;
  for (int c = c0 + t; c < c1; c += 1024) {
    int lo = 0, hi = SR;  // off[lo] <= c < off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= c) lo = mid;
      else hi = mid;
    }
    int64_t a, e;
    segment_range(q.seq_offsets, q.R, lo, q.n_positions, a, e);
    const int64_t p0 = a + (int64_t)(c - off[lo]) * kSeqChunk;
    const int64_t left = e - p0;
    const int np = left > kSeqChunk ? kSeqChunk : (int)left;
    q.desc[c] = make_int2((int)p0, (lo << 8) | np);
  }
}

}  // namespace cvr

#endif
