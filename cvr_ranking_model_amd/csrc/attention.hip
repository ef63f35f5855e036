// Query Decoding cross-attention (step B7).
//
// The CVR article (section 3.2.3) lets one query per behaviour sequence attend over that
// sequence's SwiGLU-encoded states, which serve directly as keys and values, with a
// temperature that keeps the softmax from collapsing to one-hot:
//   o = sum_t softmax_t(H[t] . q / tau) H[t]      over the valid positions t.
//
// One block of 4 waves per (candidate, sequence).  Eight lanes share a position (16
// columns each, two 16-byte loads of the bf16 row), a wave covers 8 positions and the
// block 32 per step.  Each lane group keeps an online softmax state (running max, sum of
// exponentials, weighted sum) in fp32; states are merged in a fixed butterfly order across
// lane groups and then wave by wave, so the result is bitwise reproducible.  The output is
// written in fp32 as token N+s of the token matrix.  A single pass reads each encoded state
// once.  Multiply-adds are written as explicit fmaf so that the rounding of every step is
// fixed by the source rather than by the compiler's contraction choices.
#include "device_common.h"
#include "kernels.h"

namespace cvr {

struct SoftState {
  float m, l, o[16];
};

__device__ __forceinline__ void merge_state(SoftState& a, const SoftState& b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return;  // both empty
  const float ea = expf(a.m - m), eb = expf(b.m - m);
  a.l = fmaf(a.l, ea, b.l * eb);
#pragma unroll
  for (int j = 0; j < 16; ++j) a.o[j] = fmaf(a.o[j], ea, b.o[j] * eb);
  a.m = m;
}

__device__ __forceinline__ void shfl_state(SoftState& dst, const SoftState& src, int mask) {
  dst.m = __shfl_xor(src.m, mask);
  dst.l = __shfl_xor(src.l, mask);
#pragma unroll
  for (int j = 0; j < 16; ++j) dst.o[j] = __shfl_xor(src.o[j], mask);
}

__global__ __launch_bounds__(256) void attention_kernel(const AttnParams p) {
  const int c = blockIdx.x;
  const int s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 3, sub = lane & 7;
  const int r = p.cand_req[c];
  int64_t a = p.seq_offsets[(int64_t)s * (p.R + 1) + r], e = p.seq_offsets[(int64_t)s * (p.R + 1) + r + 1];
  a = a < 0 ? 0 : (a > p.n_positions ? p.n_positions : a);
  e = e < a ? a : (e > p.n_positions ? p.n_positions : e);

  float q[16];
  {
    const float4* qp = reinterpret_cast<const float4*>(p.q + ((int64_t)s * p.n + c) * 128 + sub * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = qp[j];
      q[4 * j] = v.x;
      q[4 * j + 1] = v.y;
      q[4 * j + 2] = v.z;
      q[4 * j + 3] = v.w;
    }
  }
  SoftState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) st.o[j] = 0.f;

#pragma unroll 1
  for (int64_t t = a + wave * 8 + grp; t < e; t += 32) {
    const bf16* hp = p.H + t * 128 + sub * 16;
    const bf16x8 h0 = *reinterpret_cast<const bf16x8*>(hp);
    const bf16x8 h1 = *reinterpret_cast<const bf16x8*>(hp + 8);
    float h[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h[j] = (float)h0[j];
      h[8 + j] = (float)h1[j];
    }
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) d = fmaf(h[j], q[j], d);
    d += __shfl_xor(d, 1);
    d += __shfl_xor(d, 2);
    d += __shfl_xor(d, 4);
    const float sc = d * p.inv_tau;
    const float mn = fmaxf(st.m, sc);
    const float alpha = expf(st.m - mn);
    const float pe = expf(sc - mn);
    st.l = fmaf(st.l, alpha, pe);
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[j] = fmaf(pe, h[j], st.o[j] * alpha);
    st.m = mn;
  }
  // merge the 8 position groups of the wave (lanes differing in bits 3..5)
#pragma unroll
  for (int mask = 8; mask <= 32; mask <<= 1) {
    SoftState other;
    shfl_state(other, st, mask);
    merge_state(st, other);
  }
  __shared__ float sm[4][8][18];
  if (grp == 0) {
    sm[wave][sub][0] = st.m;
    sm[wave][sub][1] = st.l;
#pragma unroll
    for (int j = 0; j < 16; ++j) sm[wave][sub][2 + j] = st.o[j];
  }
  __syncthreads();
  if (wave == 0 && grp == 0) {
#pragma unroll 1
    for (int w = 1; w < 4; ++w) {
      SoftState o2;
      o2.m = sm[w][sub][0];
      o2.l = sm[w][sub][1];
#pragma unroll
      for (int j = 0; j < 16; ++j) o2.o[j] = sm[w][sub][2 + j];
      merge_state(st, o2);
    }
    const float inv = st.l > 0.f ? 1.0f / st.l : 0.f;
    float4* out = reinterpret_cast<float4*>(p.Y + ((int64_t)c * p.T + p.N + s) * 128 + sub * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j] = make_float4(st.o[4 * j] * inv, st.o[4 * j + 1] * inv, st.o[4 * j + 2] * inv, st.o[4 * j + 3] * inv);
  }
}

hipError_t launch_attention(const AttnParams& p, hipStream_t st) {
  if (p.n <= 0 || p.S <= 0) return hipSuccess;
  launch_k(attention_kernel, dim3(p.n, p.S), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace cvr
