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
// heads_kernel: the gate mixture, the head's first Linear and head_out in one launch.
#include <atomic>

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

// heads_kernel: 32 candidates per block of eight waves, every task: (1) the gate mixtures of each
// row, sixteen threads per row: the gate logits and every mixed expert's slice of the row are
// loaded in one batch, and each task's mixture is formed from the same registers into LDS as
// bf16 (the arithmetic of ple_gate_kernel); (2) the first Linear of every task on MFMA
// 32x32x16, wave w taking the 32-column tiles w, w+8, ... of the tasks' hidden widths laid end
// to end, one accumulation chain over k from zero, then bias, ReLU and bf16 into LDS (the
// arithmetic of the GEMM kernel's epilogue); (3) the output Linear with eight lanes per row and
// the sigmoid (the arithmetic of head_out_kernel).  Each wave's first tile's weight fragments
// and the output weights are loaded before the mixtures.  Rows past n are zero in LDS and not
// written.
constexpr int kHeadsRows = 32;
constexpr int kHeadsPitch = kHeadsMaxDim + 8;
constexpr int kHeadsWaves = 8;
__global__ __launch_bounds__(512) void heads_kernel(const HeadsParams p) {
  extern __shared__ __align__(16) bf16 heads_lds[];
  const PleGateParams& g = p.g;
  bf16* Ts = heads_lds;                                       // [K][32][pitch]
  bf16* Us = heads_lds + g.K * kHeadsRows * kHeadsPitch;      // [K][32][pitch]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = (int)blockIdx.x * kHeadsRows;
  const int rm = tid >> 4, s16 = tid & 15;  // phase 1: row rm, sixteenth s16
  const int rl = (tid >> 3) & 31, sub = tid & 7;  // phase 3 (threads 0..255): row rl, eighth `sub`
  const bool mlive = r0 + rm < g.n;
  const int lr = lane & 31, lk = 8 * (lane >> 5);
  const int ntile = p.hdim / 32;  // tiles per task
  // the first tile's weight fragments, in flight while the mixtures are formed
  constexpr int kSteps = kHeadsMaxDim / 16;
  bf16x8 wpre[kSteps];
  {
    const int k0 = wave / ntile, n0 = (wave % ntile) * 32 + lr;
    const bf16* wrow = p.W1 + (int64_t)(k0 < g.K ? k0 : 0) * p.w1_stride + (int64_t)n0 * g.edim + lk;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
      if (16 * ks < g.edim) wpre[ks] = *reinterpret_cast<const bf16x8*>(wrow + 16 * ks);
  }
  // the output weights of every task (phase 3), also in flight from the start
  bf16x8 w2v[kHeadsMaxTasks][kHeadsMaxDim / 64];
#pragma unroll
  for (int k = 0; k < kHeadsMaxTasks; ++k)
#pragma unroll
    for (int q = 0; q < kHeadsMaxDim / 64; ++q)
      if (k < g.K && 8 * sub + 64 * q < p.hdim)
        w2v[k][q] = *reinterpret_cast<const bf16x8*>(p.w2 + (int64_t)k * p.w2_stride + 8 * sub + 64 * q);
  // (1) mixtures: columns 4*s16 + 64*i of row rm, t_k = sum_e w_ke h_e in expert order
  {
    constexpr int kI = kHeadsMaxDim / 64;
    float4 h[kHeadsMaxExperts][kI];
    float lgv[kMaxTasks][kHeadsMaxExperts];
    const float* row = g.experts + (int64_t)(mlive ? r0 + rm : 0) * g.ld;
    if (mlive) {
#pragma unroll
      for (int e = 0; e < kHeadsMaxExperts; ++e)
        if (e < g.E) {
#pragma unroll
          for (int i = 0; i < kI; ++i)
            if (4 * s16 + 64 * i < g.edim) h[e][i] = *reinterpret_cast<const float4*>(row + e * g.edim + 4 * s16 + 64 * i);
        }
#pragma unroll
      for (int k = 0; k < kMaxTasks; ++k)
        if (k < g.K) {
          const int mask = g.emask[k] & ((1 << g.E) - 1);
          const float* lg = row + g.gate0 + g.goff[k];
          int r = 0;
#pragma unroll
          for (int e = 0; e < kHeadsMaxExperts; ++e)
            if ((mask >> e) & 1) lgv[k][e] = lg[r++];
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxTasks; ++k) {
      if (k >= g.K) break;
      float t[kI][4];
#pragma unroll
      for (int i = 0; i < kI; ++i) t[i][0] = t[i][1] = t[i][2] = t[i][3] = 0.f;
      if (mlive) {
        const int mask = g.emask[k] & ((1 << g.E) - 1);
        float w[kHeadsMaxExperts];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < kHeadsMaxExperts; ++e) {
          w[e] = 0.f;
          if ((mask >> e) & 1) {
            w[e] = lgv[k][e];
            mx = max_nan(mx, w[e]);
          }
        }
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < kHeadsMaxExperts; ++e) {
          w[e] = (mask >> e) & 1 ? expf(w[e] - mx) : 0.f;
          sum += w[e];
        }
        const float inv = 1.0f / sum;
#pragma unroll
        for (int e = 0; e < kHeadsMaxExperts; ++e) w[e] *= inv;
#pragma unroll
        for (int e = 0; e < kHeadsMaxExperts; ++e)
          if ((mask >> e) & 1) {
#pragma unroll
            for (int i = 0; i < kI; ++i) {
              t[i][0] += w[e] * h[e][i].x;
              t[i][1] += w[e] * h[e][i].y;
              t[i][2] += w[e] * h[e][i].z;
              t[i][3] += w[e] * h[e][i].w;
            }
          }
      }
      bf16* T = Ts + k * kHeadsRows * kHeadsPitch;
#pragma unroll
      for (int i = 0; i < kI; ++i)
        if (4 * s16 + 64 * i < g.edim) {
          bf16x4 o;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = (bf16)t[i][v];
          *reinterpret_cast<bf16x4*>(&T[rm * kHeadsPitch + 4 * s16 + 64 * i]) = o;
        }
    }
  }
  __syncthreads();
  // (2) first Linears: hidden_k[m][n] = ReLU(sum_j T_k[m][j] W1_k[n][j] + b1_k[n]), rounded to bf16
  for (int tt = wave; tt < g.K * ntile; tt += kHeadsWaves) {
    const int k = tt / ntile, n = (tt % ntile) * 32 + lr;
    const bf16* T = Ts + k * kHeadsRows * kHeadsPitch;
    const bf16* wrow = p.W1 + (int64_t)k * p.w1_stride + (int64_t)n * g.edim + lk;
    f32x16 acc = {};
    if (tt == wave) {
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks)
        if (16 * ks < g.edim)
          acc = Lowp<bf16>::mfma32(*reinterpret_cast<const bf16x8*>(&T[lr * kHeadsPitch + 16 * ks + lk]), wpre[ks], acc);
    } else {
      for (int ks = 0; ks < g.edim / 16; ++ks)
        acc = Lowp<bf16>::mfma32(*reinterpret_cast<const bf16x8*>(&T[lr * kHeadsPitch + 16 * ks + lk]),
                                 *reinterpret_cast<const bf16x8*>(wrow + 16 * ks), acc);
    }
    const float bn = p.b1[(int64_t)k * p.b1_stride + n];
    bf16* U = Us + k * kHeadsRows * kHeadsPitch;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      U[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * kHeadsPitch + n] = Lowp<bf16>::from_f32(relu_f32(acc[v] + bn));
  }
  __syncthreads();
  // (3) output Linears and sigmoids: lane `sub` takes the 8-column chunks sub, sub+8, ...
  const int c = r0 + rl;
  const bool live = tid < 8 * kHeadsRows && c < g.n;
#pragma unroll
  for (int k = 0; k < kHeadsMaxTasks; ++k) {
    if (k >= g.K) break;
    const bf16* U = Us + k * kHeadsRows * kHeadsPitch;
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < kHeadsMaxDim / 64; ++q)
      if (8 * sub + 64 * q < p.hdim) {
        const bf16x8 uv = *reinterpret_cast<const bf16x8*>(&U[rl * kHeadsPitch + 8 * sub + 64 * q]);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc += (float)uv[t] * (float)w2v[k][q][t];
      }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (live && sub == 0) {
      const float y = acc + p.b2[k][0];
      const int64_t i = (int64_t)c * g.K + k;
      p.logits[i] = y;
      p.out[i] = sigmoid_f32(y);
    }
  }
}

static size_t heads_lds_bytes(int K) { return (size_t)2 * K * kHeadsRows * kHeadsPitch * sizeof(bf16); }

bool heads_fusable(int32_t edim, int32_t hdim, int32_t n_experts, int32_t n_tasks) {
  return edim > 0 && hdim > 0 && edim % 32 == 0 && hdim % 32 == 0 && edim <= kHeadsMaxDim && hdim <= kHeadsMaxDim &&
         n_experts >= 1 && n_experts <= kHeadsMaxExperts && n_tasks >= 1 && n_tasks <= kHeadsMaxTasks;
}

hipError_t launch_heads(const HeadsParams& p, hipStream_t st) {
  if (p.g.n <= 0) return hipSuccess;
  if (!heads_fusable(p.g.edim, p.hdim, p.g.E, p.g.K)) return hipErrorInvalidValue;
  // the LDS limit is raised once per device (above the default for dynamic LDS)
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_done.load() & bit)) {
    e = hipFuncSetAttribute((const void*)heads_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)heads_lds_bytes(kHeadsMaxTasks));
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit);
  }
  launch_k(heads_kernel, dim3((unsigned)((p.g.n + kHeadsRows - 1) / kHeadsRows)), dim3(64 * kHeadsWaves),
           heads_lds_bytes(p.g.K), st, p);
  return hipGetLastError();
}

hipError_t launch_head_out(const HeadOutParams& p, hipStream_t st) {
  const int64_t total = (int64_t)p.n * p.K * 8;
  if (total <= 0) return hipSuccess;
  if (p.hdim % 8) return hipErrorInvalidValue;
  launch_k(head_out_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace cvr
