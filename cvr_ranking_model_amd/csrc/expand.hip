// Batch expansion and validation (step A0/B0), weight conversion and the synthetic table fill.
#include "chunk_plan.h"
#include "device_common.h"
#include "kernels.h"

namespace cvr {

// One thread per index i over max(n, total_bags+1, S*(R+1), R+1), 1024 per block:
//  - i < n: cand_req[i] = the request owning candidate i (largest r with cand_offsets[r] <= i);
//  - offsets checks: monotone, first 0, last equal to the declared totals.
// Every read stays inside the arrays whatever their contents.  The call's status word starts
// here: block 0 sets it to zero (no other kernel of the call has run yet, and none of this
// launch writes it), and each block stores the OR of its own checks in its block_err word, so
// the status read ORs the word and those of this launch.
__device__ __forceinline__ void expand_block(const ExpandParams& p, int64_t b, int32_t* block_bad) {
  if (threadIdx.x == 0) {
    *block_bad = 0;
    if (b == 0) p.flag[0] = 0;
  }
  __syncthreads();
  const int64_t i = b * 1024 + threadIdx.x;
  int32_t bad = 0;
  if (i < p.n) {
    int lo = 0, hi = p.R - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cand_offsets[mid] <= (int32_t)i) lo = mid; else hi = mid - 1;
    }
    p.cand_req[i] = lo;
  }
  if (i <= p.R) {
    const int32_t v = p.cand_offsets[i];
    if ((i == 0 && v != 0) || v < 0 || v > p.n) bad |= ERRF_CAND_OFFSETS;
    if (i == p.R && v != p.n) bad |= ERRF_CAND_OFFSETS;
    if (i < p.R && p.cand_offsets[i + 1] < v) bad |= ERRF_CAND_OFFSETS;
  }
  if (i <= p.total_bags) {
    const int64_t v = p.bag_offsets[i];
    if ((i == 0 && v != 0) || v < 0 || v > p.n_ids) bad |= ERRF_BAG_OFFSETS;
    if (i == p.total_bags && (p.ids_capacity ? v > p.n_ids : v != p.n_ids)) bad |= ERRF_BAG_OFFSETS;
    if (i < p.total_bags && (int64_t)p.bag_offsets[i + 1] < v) bad |= ERRF_BAG_OFFSETS;
  }
  if (p.seq_offsets != nullptr && i < (int64_t)p.S * (p.R + 1)) {
    // The [S][R+1] array read as one list must be non-decreasing: each sequence's segments in
    // request order, and sequence s ending at or before sequence s+1 begins.  Segments are
    // then disjoint inside [0, n_positions], so every position is encoded by one sequence's
    // weights and the chunk count stays within n_positions / 32 + S * R.
    const int64_t v = p.seq_offsets[i];
    if (v < 0 || v > p.n_positions) bad |= ERRF_SEQ_OFFSETS;
    if (i + 1 < (int64_t)p.S * (p.R + 1) && (int64_t)p.seq_offsets[i + 1] < v) bad |= ERRF_SEQ_OFFSETS;
  }
  if (bad) atomicOr(block_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) p.block_err[b] = *block_bad;
}

__global__ __launch_bounds__(1024) void expand_kernel(const ExpandParams p) {
  __shared__ int32_t block_bad;
  expand_block(p, blockIdx.x, &block_bad);
}

// Expansion and chunk plan side by side: blocks [0, nexp) expand, the rest plan (they read only
// the sequence offsets, which no kernel of the call writes).  The plan's offset table sits in
// dynamic LDS (S*R+1 entries).
__global__ __launch_bounds__(1024) void front_kernel(const ExpandParams p, int32_t nexp, const PlanParams q) {
  extern __shared__ int32_t plan_off[];
  __shared__ int32_t block_bad;
  __shared__ long long wsum[16];
  if ((int)blockIdx.x < nexp) expand_block(p, blockIdx.x, &block_bad);
  else chunk_plan_block(q, (int)blockIdx.x - nexp, (int)gridDim.x - nexp, plan_off, wsum);
}

int64_t expand_blocks(int64_t n, int64_t total_bags, int64_t R, int64_t S) {
  int64_t work = n;
  if (total_bags + 1 > work) work = total_bags + 1;
  if (R + 1 > work) work = R + 1;
  if (S * (R + 1) > work) work = S * (R + 1);
  return (work + 1023) / 1024;
}

hipError_t launch_expand(const ExpandParams& p, int64_t blocks, hipStream_t st) {
  const int64_t need = expand_blocks(p.n, p.total_bags, p.R, p.seq_offsets ? p.S : 0);
  if (blocks < need || blocks > INT32_MAX) return hipErrorInvalidValue;
  launch_k(expand_kernel, dim3((unsigned)blocks), dim3(1024), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_front(const ExpandParams& p, int64_t blocks, const PlanParams& q, hipStream_t st) {
  const int64_t need = expand_blocks(p.n, p.total_bags, p.R, p.seq_offsets ? p.S : 0);
  if (blocks < need || (int64_t)q.S * q.R > kPlanMaxSegs) return hipErrorInvalidValue;
  const int64_t total = blocks + chunk_plan_blocks(q.max_chunks);
  if (total > INT32_MAX) return hipErrorInvalidValue;
  launch_k(front_kernel, dim3((unsigned)total), dim3(1024), (size_t)((int64_t)q.S * q.R + 1) * 4, st, p,
           (int32_t)blocks, q);
  return hipGetLastError();
}

// ------------------------------------------------------------------ conversion
template <typename T>
__global__ void convert_kernel(const float* __restrict__ src, T* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = Lowp<T>::from_f32(src[i]);
}

hipError_t launch_convert(const float* src, void* dst, int64_t n, int lowp, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (lowp == 0)
    launch_k(convert_kernel<f16>, dim3((unsigned)blocks), dim3(256), 0, st, src, (f16*)dst, n);
  else
    launch_k(convert_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, st, src, (bf16*)dst, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ synthetic table fill
// Element i gets (k - 2^23) * step (fp64 product, rounded to fp32), k = top 24 bits of the
// (i+1)-th SplitMix64 output for the given seed.  Four consecutive elements per thread.
__global__ void fill_kernel(float* __restrict__ t, int64_t quads, uint64_t seed, double step) {
  const uint64_t gamma = 0x9E3779B97F4A7C15ull;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += (int64_t)gridDim.x * blockDim.x) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t i = (uint64_t)(q * 4 + j);
      const uint64_t x = splitmix64_mix(seed + (i + 1) * gamma);
      const int64_t k = (int64_t)(x >> 40) - (int64_t)(1 << 23);
      v[j] = (float)((double)k * step);
    }
    *reinterpret_cast<float4*>(t + q * 4) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

hipError_t launch_fill_table(float* t, int64_t total, uint64_t seed, double step, hipStream_t st) {
  const int64_t quads = total / 4;
  int64_t blocks = (quads + 255) / 256;
  if (blocks > 262144) blocks = 262144;
  if (blocks > 0) launch_k(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, t, quads, seed, step);
  return hipGetLastError();
}

}  // namespace cvr
