// Launch interfaces of the libcvr kernels (host side).  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cvr {

// Device error flag bits (OR-ed into the workspace's status word).
enum : int32_t {
  ERRF_CAND_OFFSETS = 1,
  ERRF_BAG_OFFSETS = 2,
  ERRF_ID_RANGE = 4,
  ERRF_SEQ_OFFSETS = 8,
  ERRF_SEQ_ID_RANGE = 16,
};

constexpr int kMaxGatherFeatures = 32;
constexpr int kSeqChunk = 64;  // positions per SwiGLU work item (never spanning two sequences)
constexpr int kMaxASegments = 4;

// ---------------------------------------------------------------- expand (A0/B0)
struct ExpandParams {
  const int32_t* cand_offsets;  // [R+1]
  int32_t R;
  int32_t n;
  const int32_t* bag_offsets;   // [total_bags+1]
  int64_t total_bags;
  int64_t n_ids;
  const int32_t* seq_offsets;   // [S][R+1] or null
  int32_t S;
  int64_t n_positions;
  int32_t* cand_req;            // [n] out
  int32_t* flag;                // status word (cleared by this launch's first block before use)
};
hipError_t launch_clear_flag(int32_t* flag, hipStream_t st);
hipError_t launch_expand(const ExpandParams& p, hipStream_t st);

// ---------------------------------------------------------------- gather + mean-pool (A1-A2/B1)
struct GatherFeature {
  const float* table;
  int64_t rows;
  int32_t dim;          // multiple of 4, <= 256
  int32_t nbags;        // bags of this feature in the batch (R or n)
  int64_t bag_base;     // index of its first bag in bag_offsets
  void* out;            // low-precision matrix; row = local bag index
  int32_t ldo;          // elements per output row
  int32_t col;          // first output column
  float* dbg;           // fp32 pooled [nbags][dim] or null
  int32_t block_begin;  // first block of this feature in the launch
  int32_t pad_;
};
struct GatherParams {
  GatherFeature f[kMaxGatherFeatures];
  int32_t nf;
  int32_t total_blocks;
  const int32_t* bag_offsets;
  const int32_t* ids;
  int64_t n_ids;
  float clamp;
  int32_t lowp;         // 0 fp16, 1 bf16
  int32_t* flag;
};
// Fills block_begin/total_blocks and launches.
hipError_t launch_gather_pool(GatherParams& p, hipStream_t st);

// ---------------------------------------------------------------- GEMM (MFMA)
// C(m, n) = epilogue( sum_k A(m, k) * W(n, k) + bias(n) ) for a group index g.
// A(m, k): K is split into segments; in segment s (k_begin..k_end) with kk = k - k_begin + col0,
//   A(m, k) = seg.ptr[g*seg.gstride + row*seg.ld + (kk/8)*seg.kstride8 + kk%8], row = rowmap ? rowmap[m] : m.
// W(n, k) = W[g*w_gstride + n*K + k].   C(m, n) at C[g*c_gstride + m*ldc + (n/8)*c_nstride8 + n%8];
// the optional residual R uses the same addressing as C.
struct ASeg {
  const void* ptr;
  const int32_t* rowmap;
  int64_t ld;
  int64_t gstride;
  int32_t k_end;
  int32_t kstride8;
  int32_t col0;
  int32_t pad_;
};
struct GemmParams {
  int32_t M, N, K;
  int32_t groups;
  int32_t nseg;
  ASeg seg[kMaxASegments];
  const void* W;
  int64_t w_gstride;
  const float* bias;
  int64_t bias_gstride;
  void* C;
  int64_t ldc;
  int64_t c_gstride;
  int32_t c_nstride8;
  const void* R;        // residual (same type and addressing as C) or null
  int32_t relu;
  int32_t out_f32;      // 1: C is fp32, else the low-precision type
};
hipError_t launch_gemm(const GemmParams& p, int lowp, hipStream_t st);

// ---------------------------------------------------------------- DLRM output (A4)
// z[m] = sum_k H[m][k] * w[k] + b  (fp32 accumulation), out[m] = sigmoid(z[m]).
hipError_t launch_dlrm_output(const void* H, int32_t M, int32_t K, const void* w, const float* b,
                              float* logits, float* out, int lowp, hipStream_t st);

// ---------------------------------------------------------------- fill (input generator)
hipError_t launch_fill_table(float* t, int64_t total, uint64_t seed, double step, hipStream_t st);

// ---------------------------------------------------------------- weight packing
// fp32 -> low precision, elementwise (n elements).
hipError_t launch_convert(const float* src, void* dst, int64_t n, int lowp, hipStream_t st);

}  // namespace cvr
