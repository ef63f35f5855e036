// Query Decoding cross-attention (step B7).
//
// The CVR article (section 3.2.3) lets one query per behaviour sequence attend over that
// sequence's SwiGLU-encoded states, which serve directly as keys and values, with a
// temperature that keeps the softmax from collapsing to one-hot:
//   o = sum_t softmax_t(H[t] . q / tau) H[t]      over the valid positions t.
//
// One block of 4 waves per (candidate, sequence).  Eight lanes share a position: lane `sub`
// holds columns 8*sub .. 8*sub+7 and 64 + 8*sub .. 64 + 8*sub + 7, so each 16-byte load of a
// wave reads one whole 128-byte half row for each of its 8 positions; a wave covers 8 positions
// and the block 32 per step, and each lane group loads its next position before it works on
// the current one.  Each lane group keeps an online softmax state (running max, sum of
// exponentials, weighted sum) in fp32; states are merged in a fixed butterfly order across
// lane groups and then wave by wave, so the result is bitwise reproducible.  The output is
// written in fp32 as token N+s of the token matrix.  A single pass reads each encoded state
// once.  Multiply-adds are written as explicit fmaf so that the rounding of every step is
// fixed by the source rather than by the compiler's contraction choices.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace cvr {

struct SoftState {
  float m, l, o[16];
};

__device__ __forceinline__ void merge_state(SoftState& a, const SoftState& b) {
  const float m = max_nan(a.m, b.m);
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

template <bool kNT>
__global__ __launch_bounds__(256) void attention_kernel(const AttnParams p) {
  const int c = blockIdx.x;
  const int s = p.S - 1 - (int)blockIdx.y;  // the last (longest) sequence first: a shorter tail
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 3, sub = lane & 7;
  const int r = p.cand_req[c];
  int64_t a = p.seq_offsets[(int64_t)s * (p.R + 1) + r], e = p.seq_offsets[(int64_t)s * (p.R + 1) + r + 1];
  a = a < 0 ? 0 : (a > p.n_positions ? p.n_positions : a);
  e = e < a ? a : (e > p.n_positions ? p.n_positions : e);

  // q[0..7] = columns 8*sub.., q[8..15] = columns 64 + 8*sub..
  float q[16];
  {
    const float* qrow = p.q + ((int64_t)s * p.n + c) * 128;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float4* qp = reinterpret_cast<const float4*>(qrow + 64 * hf + sub * 8);
      const float4 v0 = qp[0], v1 = qp[1];
      q[8 * hf + 0] = v0.x;
      q[8 * hf + 1] = v0.y;
      q[8 * hf + 2] = v0.z;
      q[8 * hf + 3] = v0.w;
      q[8 * hf + 4] = v1.x;
      q[8 * hf + 5] = v1.y;
      q[8 * hf + 6] = v1.z;
      q[8 * hf + 7] = v1.w;
    }
  }
  SoftState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) st.o[j] = 0.f;

  // the row of position t: columns 8*sub.. and 64 + 8*sub..  (kNT: nontemporal loads, for
  // states that outsize the last-level cache)
  auto load_row = [&](int64_t t, bf16x8& h0, bf16x8& h1) {
    const bf16x8* hp = reinterpret_cast<const bf16x8*>(p.H + t * 128 + sub * 8);
    if constexpr (kNT) {
      h0 = __builtin_nontemporal_load(hp);
      h1 = __builtin_nontemporal_load(hp + 8);
    } else {
      h0 = hp[0];
      h1 = hp[8];
    }
  };
  int64_t t = a + wave * 8 + grp;
  bf16x8 n0, n1;
  if (t < e) load_row(t, n0, n1);
#pragma unroll 1
  for (; t < e; t += 32) {
    const bf16x8 h0 = n0, h1 = n1;
    if (t + 32 < e) load_row(t + 32, n0, n1);
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
    const float mn = max_nan(st.m, sc);
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
    const float inv = st.l == 0.f ? 0.f : 1.0f / st.l;  // an empty sequence gives 0; NaN passes
    float* orow = p.Y + ((int64_t)c * p.T + p.N + s) * 128;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float4* out = reinterpret_cast<float4*>(orow + 64 * hf + sub * 8);
      out[0] = make_float4(st.o[8 * hf] * inv, st.o[8 * hf + 1] * inv, st.o[8 * hf + 2] * inv, st.o[8 * hf + 3] * inv);
      out[1] = make_float4(st.o[8 * hf + 4] * inv, st.o[8 * hf + 5] * inv, st.o[8 * hf + 6] * inv, st.o[8 * hf + 7] * inv);
    }
  }
}

// ---------------------------------------------------------------- many candidates per request
// When a request carries many candidates, their queries share the request's keys and values,
// so attention over one sequence is two dense products per request and runs on MFMA:
//   S^T = H Q^T / tau  (positions x candidates),  O^T = H^T softmax(S)^T  (dims x candidates).
// One block per (tile of 32 consecutive candidates, sequence): its four waves take every fourth
// block of 32 of the request's positions (loading the next one while computing), each with an
// online softmax (fp32 state per candidate, the candidate's lane keeps it), and the four
// states are merged in wave order at the end.
// Queries are split into a bf16 high part and a bf16 remainder, and so are the softmax
// weights, so both products keep about 16 bits of the fp32 operand (the encoded states are
// bf16 already).  A tile that straddles requests takes one pass per request, with the other
// candidates' columns masked.
//
// MFMA 32x32x16 layouts: lane l holds A[l%32][8(l/32)..+7] and B[8(l/32)..+7][l%32]; result
// element v sits at row 8(v/4) + 4(l/32) + v%4, column l%32.  In S^T a lane therefore holds 16
// positions of candidate l%32 (the other 16 are in lane l^32), and the weights it feeds as the
// B operand of the value product cover the positions of k-step kk in the order
// 16kk + 8(i/4) + 4(l/32) + i%4, i = 0..7 -- the states are stored transposed in LDS in that
// order (slot = position with bits 2 and 3 swapped).
constexpr int kMqPitch = 32 + 8;  // bf16 per transposed row: 16-byte reads of 16 rows hit distinct banks

__global__ __launch_bounds__(256) void attention_mq_kernel(const AttnParams p) {
  __shared__ __align__(16) bf16 Ht[4][128 * kMqPitch];
  __shared__ float Ms[3][2][32];        // waves 1-3: running max and sum per candidate
  __shared__ float4 Os[3][16][64];      // waves 1-3: weighted sums, in the lanes' own layout
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ntiles = (p.n + 31) / 32;
  const int task = blockIdx.x;
  const int s = p.S - 1 - task / ntiles;  // longest sequences first
  const int c0 = (task % ntiles) * 32;
  const int lr = lane & 31, hf = lane >> 5, h8 = hf * 8;
  const bool cvalid = c0 + lr < p.n;
  const int cl = cvalid ? c0 + lr : p.n - 1;
  const int myreq = p.cand_req[cl];
  bf16* ht = Ht[wave];

  // B operand of S^T: Q[candidate lr][16k + 8(l/32) .. +7], as high and remainder parts
  bf16x8 qh[8], ql[8];
  {
    const float* qrow = p.q + ((int64_t)s * p.n + cl) * 128;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 x0 = *reinterpret_cast<const float4*>(qrow + 16 * k + h8);
      const float4 x1 = *reinterpret_cast<const float4*>(qrow + 16 * k + h8 + 4);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qh[k][i] = (bf16)xs[i];
        ql[k][i] = (bf16)(xs[i] - (float)qh[k][i]);
      }
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int slot = (lr & ~12) | ((lr & 4) << 1) | ((lr & 8) >> 1);  // this lane's position -> LDS slot

  // One block of 32 positions starting at t0 (rows already in hv).
  auto block = [&](const bf16x8 (&hv)[8], int64_t t0, int64_t e, bool active) {
    f32x16 sc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sc = Lowp<bf16>::mfma32(hv[k], qh[k], sc);
      sc = Lowp<bf16>::mfma32(hv[k], ql[k], sc);
    }
    // transposed copy of the block for the value product
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) ht[(16 * k + h8 + i) * kMqPitch + slot] = hv[k][i];
    // online softmax for candidate lr over the block's positions
    float x[16];
    float bm = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t pos = t0 + 8 * (v >> 2) + 4 * hf + (v & 3);
      x[v] = active && pos < e ? sc[v] * p.inv_tau : -INFINITY;
      bm = max_nan(bm, x[v]);
    }
    bm = max_nan(bm, __shfl_xor(bm, 32));
    const float mn = max_nan(m, bm);
    const float alpha = mn == -INFINITY ? 1.f : expf(m - mn);
    float pv[16], ps = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      pv[v] = x[v] == -INFINITY ? 0.f : expf(x[v] - mn);
      ps += pv[v];
    }
    ps += __shfl_xor(ps, 32);
    l = fmaf(l, alpha, ps);
    m = mn;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][v] *= alpha;
    // O^T += H^T P^T: A = transposed states (dims x slots), B = weights (slots x candidates)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 ph, pl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ph[i] = (bf16)pv[8 * kk + i];
        pl[i] = (bf16)(pv[8 * kk + i] - (float)ph[i]);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&ht[(32 * dt + lr) * kMqPitch + 16 * kk + h8]);
        acc[dt] = Lowp<bf16>::mfma32(av, ph, acc[dt]);
        acc[dt] = Lowp<bf16>::mfma32(av, pl, acc[dt]);
      }
    }
  };
  // A operand rows: the state row of position t0 + lr (past the end: the last row, masked)
  auto load = [&](bf16x8 (&hv)[8], int64_t t0, int64_t e) {
    const int64_t tr = t0 + lr < e ? t0 + lr : e - 1;
#pragma unroll
    for (int k = 0; k < 8; ++k) hv[k] = *reinterpret_cast<const bf16x8*>(p.H + tr * 128 + 16 * k + h8);
  };

  const int r_first = p.cand_req[c0], r_last = p.cand_req[min(c0 + 31, p.n - 1)];
#pragma unroll 1
  for (int r = r_first; r <= r_last; ++r) {
    const bool active = cvalid && myreq == r;
    if (!__any(active)) continue;
    int64_t a = p.seq_offsets[(int64_t)s * (p.R + 1) + r], e = p.seq_offsets[(int64_t)s * (p.R + 1) + r + 1];
    a = a < 0 ? 0 : (a > p.n_positions ? p.n_positions : a);
    e = e < a ? a : (e > p.n_positions ? p.n_positions : e);
    // the waves take every fourth block of 32 positions; each loads its next block early
    int64_t t0 = a + 32 * wave;
    if (t0 >= e) continue;
    bf16x8 hv[8], hn[8];
    load(hv, t0, e);
#pragma unroll 1
    while (true) {
      const int64_t tn = t0 + 128;
      if (tn < e) load(hn, tn, e);
      block(hv, t0, e, active);
      if (tn >= e) break;
      t0 = tn;
#pragma unroll
      for (int k = 0; k < 8; ++k) hv[k] = hn[k];
    }
  }
  // merge the waves' states in wave order
  if (wave > 0) {
    if (lane < 32) {
      Ms[wave - 1][0][lr] = m;
      Ms[wave - 1][1][lr] = l;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        Os[wave - 1][4 * dt + v4][lane] =
            make_float4(acc[dt][4 * v4], acc[dt][4 * v4 + 1], acc[dt][4 * v4 + 2], acc[dt][4 * v4 + 3]);
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll 1
  for (int w = 0; w < 3; ++w) {
    const float mw = Ms[w][0][lr], lw = Ms[w][1][lr];
    const float mn = max_nan(m, mw);
    if (mn == -INFINITY) continue;
    const float a0 = expf(m - mn), aw = expf(mw - mn);
    l = fmaf(l, a0, lw * aw);
    m = mn;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const float4 o = Os[w][4 * dt + v4][lane];
        acc[dt][4 * v4] = fmaf(acc[dt][4 * v4], a0, o.x * aw);
        acc[dt][4 * v4 + 1] = fmaf(acc[dt][4 * v4 + 1], a0, o.y * aw);
        acc[dt][4 * v4 + 2] = fmaf(acc[dt][4 * v4 + 2], a0, o.z * aw);
        acc[dt][4 * v4 + 3] = fmaf(acc[dt][4 * v4 + 3], a0, o.w * aw);
      }
  }
  if (cvalid) {
    const float inv = l == 0.f ? 0.f : 1.0f / l;  // an empty sequence gives 0; NaN passes
    float* out = p.Y + ((int64_t)(c0 + lr) * p.T + p.N + s) * 128;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        *reinterpret_cast<float4*>(out + 32 * dt + 8 * v4 + 4 * hf) =
            make_float4(acc[dt][4 * v4] * inv, acc[dt][4 * v4 + 1] * inv, acc[dt][4 * v4 + 2] * inv,
                        acc[dt][4 * v4 + 3] * inv);
  }
}

bool attention_many_candidates(int32_t n, int32_t R) { return (int64_t)n >= 16 * (int64_t)R; }

hipError_t launch_attention(const AttnParams& p, hipStream_t st) {
  if (p.n <= 0 || p.S <= 0) return hipSuccess;
  if (p.mq) {
    const int64_t tasks = (int64_t)((p.n + 31) / 32) * p.S;
    launch_k(attention_mq_kernel, dim3((unsigned)tasks), dim3(256), 0, st, p);
  } else {
    if (p.nt)
      launch_k(attention_kernel<true>, dim3(p.n, p.S), dim3(256), 0, st, p);
    else
      launch_k(attention_kernel<false>, dim3(p.n, p.S), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace cvr
