// Prediction level of the CVR model (steps B10-B11) around the expert and head GEMMs.
//
// The CVR article (section 3.2.4) predicts each scenario's pCVR with PLE + MLP heads: three
// experts that are single fully-connected layers, mixed per task, and heads of two
// fully-connected layers with a nonlinearity.  The expert Linear+ReLU and the first head
// Linear+ReLU run as MFMA GEMMs; this file holds the two small pieces between and after:
//
// ple_gate_kernel (one wave per candidate): the per-task gate logits W_g z + b_g over the
//   flattened token matrix z (rounded to bf16 as a Linear input; fp32 dot products with a
//   fixed-order wave reduction), a softmax in fp32 over the experts the task mixes (all of
//   them when the experts are shared; its own plus the shared ones for PLE with
//   task-specific experts), and the gated mixture t_k = sum_e g_ke h_e of those experts'
//   fp32 outputs, rounded to bf16 (it is the input of the head's first Linear).
// head_out_kernel (one thread per candidate and task): y = w2 . u + b2 with fp32
//   accumulation and the fp32 sigmoid; writes out[c * n_tasks + k].
#include "device_common.h"
#include "kernels.h"

namespace cvr {

__global__ __launch_bounds__(256) void ple_gate_kernel(const PleGateParams p) {
  const int c = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= p.n) return;
  const float* z = p.Z + (int64_t)c * p.zdim;
  // logit[k * E + e] for the experts task k mixes; the others take no part.
  float logit[kMaxTasks * kMaxExperts];
#pragma unroll 1
  for (int k = 0; k < p.K; ++k) {
    int row = 0;
#pragma unroll 1
    for (int e = 0; e < p.E; ++e) {
      if (!((p.emask[k] >> e) & 1)) continue;
      const bf16* w = p.wg[k] + (int64_t)row * p.zdim;
      float acc = 0.f;
      for (int j = lane * 8; j < p.zdim; j += 512) {
        const float4 z0 = *reinterpret_cast<const float4*>(z + j);
        const float4 z1 = *reinterpret_cast<const float4*>(z + j + 4);
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        const bf16x8 wv = *reinterpret_cast<const bf16x8*>(w + j);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += (float)(bf16)zv[u] * (float)wv[u];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
      logit[k * p.E + e] = acc + p.bg[k][row];
      ++row;
    }
  }
  for (int k = 0; k < p.K; ++k) {
    const int mask = p.emask[k];
    float mx = -INFINITY;
    for (int e = 0; e < p.E; ++e)
      if ((mask >> e) & 1) mx = fmaxf(mx, logit[k * p.E + e]);
    float g[kMaxExperts], sum = 0.f;
    for (int e = 0; e < p.E; ++e) {
      g[e] = (mask >> e) & 1 ? expf(logit[k * p.E + e] - mx) : 0.f;
      sum += g[e];
    }
    const float inv = 1.0f / sum;
    for (int e = 0; e < p.E; ++e) g[e] *= inv;
    for (int j = lane; j < p.edim; j += 64) {
      float t = 0.f;
      for (int e = 0; e < p.E; ++e)
        if ((mask >> e) & 1) t += g[e] * p.experts[(int64_t)c * p.E * p.edim + e * p.edim + j];
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
