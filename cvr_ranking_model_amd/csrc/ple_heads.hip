// Prediction level of the CVR model (steps B10-B11) around the expert and head GEMMs.
//
// The CVR article (section 3.2.4) predicts each scenario's pCVR with PLE + MLP heads: three
// experts that are single fully-connected layers, mixed per task, and heads of two
// fully-connected layers with a nonlinearity.  The expert Linear+ReLU and the first head
// Linear+ReLU run as MFMA GEMMs; this file holds the two small pieces between and after:
//
// ple_gate_kernel (one wave per candidate): the gate logits W_g z + b_g come from the expert
//   GEMM (the gate rows sit after the expert rows, so one MFMA pass over z yields both); this
//   kernel takes a softmax in fp32 over the experts each task mixes (all of them when the
//   experts are shared; its own plus the shared ones for PLE with task-specific experts) and
//   forms the gated mixture t_k = sum_e g_ke h_e of those experts' fp32 outputs, rounded to
//   bf16 (it is the input of the head's first Linear).
// head_out_kernel (eight lanes per candidate and task): y = w2 . u + b2 with fp32
//   accumulation and the fp32 sigmoid; writes out[c * n_tasks + k].
#include "device_common.h"
#include "kernels.h"

namespace cvr {

__global__ __launch_bounds__(256) void ple_gate_kernel(const PleGateParams p) {
  const int c = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= p.n) return;
  const float* row = p.experts + (int64_t)c * p.ld;  // 128-byte aligned rows
  for (int k = 0; k < p.K; ++k) {
    const int mask = p.emask[k] & ((1 << p.E) - 1);
    const float* lg = row + p.gate0 + p.goff[k];  // one logit per expert the task mixes, in expert order
    float g[kMaxExperts];
    float mx = -INFINITY;
    int r = 0;
#pragma unroll
    for (int e = 0; e < kMaxExperts; ++e) {
      g[e] = 0.f;
      if ((mask >> e) & 1) {
        g[e] = lg[r++];
        mx = max_nan(mx, g[e]);
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxExperts; ++e) {
      g[e] = (mask >> e) & 1 ? expf(g[e] - mx) : 0.f;
      sum += g[e];
    }
    const float inv = 1.0f / sum;
#pragma unroll
    for (int e = 0; e < kMaxExperts; ++e) g[e] *= inv;
    // four consecutive columns per lane (16-byte loads of each expert's output, 8-byte stores)
    for (int j = 4 * lane; j < p.edim; j += 256) {
      float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < kMaxExperts; ++e)
        if ((mask >> e) & 1) {
          const float4 h = *reinterpret_cast<const float4*>(row + e * p.edim + j);
          t[0] += g[e] * h.x;
          t[1] += g[e] * h.y;
          t[2] += g[e] * h.z;
          t[3] += g[e] * h.w;
        }
      bf16x4 o;
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = (bf16)t[v];
      *reinterpret_cast<bf16x4*>(p.task_in + ((int64_t)k * p.n + c) * p.edim + j) = o;
    }
  }
}

hipError_t launch_ple_gate(const PleGateParams& p, hipStream_t st) {
  if (p.n <= 0) return hipSuccess;
  launch_k(ple_gate_kernel, dim3((p.n + 3) / 4), dim3(256), 0, st, p);
  return hipGetLastError();
}

// Eight lanes per (candidate, task): lane `sub` takes the 8-column chunks sub, sub+8, ... of the
// hidden row, accumulating in chunk order, and the eight partial sums are combined by a fixed
// butterfly (deterministic).
__global__ __launch_bounds__(256) void head_out_kernel(const HeadOutParams p) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int sub = (int)(gi & 7);
  const int64_t i = gi >> 3;
  const bool live = i < (int64_t)p.n * p.K;
  const int c = live ? (int)(i / p.K) : 0, k = live ? (int)(i % p.K) : 0;
  const bf16* u = p.U + ((int64_t)k * p.n + c) * p.hdim;
  const bf16* w = p.w2 + (int64_t)k * p.w2_stride;
  float acc = 0.f;
  if (live)
    for (int j = 8 * sub; j < p.hdim; j += 64) {
      const bf16x8 uv = *reinterpret_cast<const bf16x8*>(u + j);
      const bf16x8 wv = *reinterpret_cast<const bf16x8*>(w + j);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc += (float)uv[t] * (float)wv[t];
    }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (live && sub == 0) {
    const float y = acc + p.b2[k][0];
    p.logits[i] = y;
    p.out[i] = sigmoid_f32(y);
  }
}

hipError_t launch_head_out(const HeadOutParams& p, hipStream_t st) {
  const int64_t total = (int64_t)p.n * p.K * 8;
  if (total <= 0) return hipSuccess;
  if (p.hdim % 8) return hipErrorInvalidValue;
  launch_k(head_out_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace cvr
