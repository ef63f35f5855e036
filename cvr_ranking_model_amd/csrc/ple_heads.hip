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
// head_out_kernel (one thread per candidate and task): y = w2 . u + b2 with fp32
//   accumulation and the fp32 sigmoid; writes out[c * n_tasks + k].
#include "device_common.h"
#include "kernels.h"

namespace cvr {

__global__ __launch_bounds__(256) void ple_gate_kernel(const PleGateParams p) {
  const int c = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= p.n) return;
  const float* row = p.experts + (int64_t)c * p.ld;
  for (int k = 0; k < p.K; ++k) {
    const int mask = p.emask[k];
    const float* lg = row + p.gate0 + p.goff[k];  // one logit per expert the task mixes
    float logit[kMaxExperts];
    float mx = -INFINITY;
    int r = 0;
    for (int e = 0; e < p.E; ++e)
      if ((mask >> e) & 1) {
        logit[e] = lg[r++];
        mx = max_nan(mx, logit[e]);
      }
    float g[kMaxExperts], sum = 0.f;
    for (int e = 0; e < p.E; ++e) {
      g[e] = (mask >> e) & 1 ? expf(logit[e] - mx) : 0.f;
      sum += g[e];
    }
    const float inv = 1.0f / sum;
    for (int e = 0; e < p.E; ++e) g[e] *= inv;
    for (int j = lane; j < p.edim; j += 64) {
      float t = 0.f;
      for (int e = 0; e < p.E; ++e)
        if ((mask >> e) & 1) t += g[e] * row[e * p.edim + j];
      p.task_in[((int64_t)k * p.n + c) * p.edim + j] = (bf16)t;
    }
  }
}

hipError_t launch_ple_gate(const PleGateParams& p, hipStream_t st) {
  if (p.n <= 0) return hipSuccess;
  launch_k(ple_gate_kernel, dim3((p.n + 3) / 4), dim3(256), 0, st, p);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void head_out_kernel(const HeadOutParams p) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.n * p.K) return;
  const int c = i / p.K, k = i % p.K;
  const bf16* u = p.U + ((int64_t)k * p.n + c) * p.hdim;
  const bf16* w = p.w2 + (int64_t)k * p.w2_stride;
  float acc = 0.f;
  for (int j = 0; j < p.hdim; j += 8) {
    const bf16x8 uv = *reinterpret_cast<const bf16x8*>(u + j);
    const bf16x8 wv = *reinterpret_cast<const bf16x8*>(w + j);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc += (float)uv[t] * (float)wv[t];
  }
  const float y = acc + p.b2[k][0];
  p.logits[i] = y;
  p.out[i] = sigmoid_f32(y);
}

hipError_t launch_head_out(const HeadOutParams& p, hipStream_t st) {
  const int total = p.n * p.K;
  if (total <= 0) return hipSuccess;
  launch_k(head_out_kernel, dim3((total + 255) / 256), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace cvr
