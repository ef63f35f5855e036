// Dense contractions on the gfx950 matrix cores (steps A3, B2, B6, B8, B10, B11).
//
// C = epilogue(A * W^T + bias) with fp16/bf16 operands and fp32 accumulation,
// using the 32x32x16 MFMA.  Both operands are K-contiguous (activations [M][K],
// Linear weights [N][K]), which is exactly the per-lane layout the MFMA wants
// (8 consecutive k per lane), so every global load and every LDS read is one
// 16-byte access.  A block of 4 waves computes a BM x BN tile; the K loop
// stages 32-wide slices of both operands through LDS (double-buffered, one
// barrier per slice, rows padded to 80 bytes so the 16-byte fragment reads of a
// quarter-wave hit distinct banks).  Blocks are renumbered so that the tiles
// sharing one A row-block run on the same XCD and reuse it from that XCD's L2.
//
// The A operand may be assembled from up to four K-segments, each with its own
// base, row stride, optional row map and 8-element chunk stride.  This lets the
// first Linear read the request-side inputs through the candidate->request map
// (the "lazy repeat" of the user side, CVR article section 3.4.5), and lets the
// token mixer read and write its Split/Revert layouts without a transpose pass.
#include "device_common.h"
#include "kernels.h"

namespace cvr {

constexpr int kBK = 32;
constexpr int kPitch = kBK + 8;  // elements per LDS row

template <typename T, int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams p) {
  typedef typename Lowp<T>::vec8 V8;
  constexpr int WTM = BM / WGM;
  constexpr int WTN = BN / WGN;
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int AQ = BM * kBK / 8 / 256;  // 16-byte A chunks per thread per K slice
  constexpr int BQ = BN * kBK / 8 / 256;
  static_assert(WGM * WGN == 4, "4 waves");
  static_assert(AQ >= 1 && BQ >= 1, "tile too small");

  __shared__ __align__(16) T As[2][BM * kPitch];
  __shared__ __align__(16) T Bs[2][BN * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN;
  const int wn = wave % WGN;
  const int g = blockIdx.y;

  // XCD-aware renumbering: hardware dispatch puts block b on XCD b % 8.
  const int ntn = (p.N + BN - 1) / BN;
  const int total = gridDim.x;
  int lb = blockIdx.x;
  if ((total & 7) == 0) lb = (lb & 7) * (total >> 3) + (lb >> 3);
  const int m0 = (lb / ntn) * BM;
  const int n0 = (lb % ntn) * BN;

  const T* Wg = reinterpret_cast<const T*>(p.W) + (int64_t)g * p.w_gstride;

  u32x4 ra[AQ], rb[BQ];

  auto load_slice = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AQ; ++i) {
      const int q = tid + i * 256;
      const int r = q >> 2;
      const int k = k0 + (q & 3) * 8;
      int m = m0 + r;
      m = m < p.M ? m : p.M - 1;
      int s = 0, kb = 0;
#pragma unroll 1
      for (; s < p.nseg - 1; ++s) {
        if (k < p.seg[s].k_end) break;
        kb = p.seg[s].k_end;
      }
      const ASeg& S = p.seg[s];
      const int kk = k - kb + S.col0;
      const int64_t row = S.rowmap ? (int64_t)S.rowmap[m] : (int64_t)m;
      const int64_t eoff = (int64_t)g * S.gstride + row * S.ld + (int64_t)(kk >> 3) * S.kstride8;
      if (S.f32) {
        const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(S.ptr) + eoff);
        const float4 x0 = src[0], x1 = src[1];
        V8 v;
        v[0] = Lowp<T>::from_f32(x0.x); v[1] = Lowp<T>::from_f32(x0.y);
        v[2] = Lowp<T>::from_f32(x0.z); v[3] = Lowp<T>::from_f32(x0.w);
        v[4] = Lowp<T>::from_f32(x1.x); v[5] = Lowp<T>::from_f32(x1.y);
        v[6] = Lowp<T>::from_f32(x1.z); v[7] = Lowp<T>::from_f32(x1.w);
        ra[i] = *reinterpret_cast<const u32x4*>(&v);
      } else {
        ra[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(S.ptr) + eoff);
      }
    }
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      const int q = tid + i * 256;
      const int r = q >> 2;
      int n = n0 + r;
      n = n < p.N ? n : p.N - 1;
      rb[i] = *reinterpret_cast<const u32x4*>(Wg + (int64_t)n * p.K + k0 + (q & 3) * 8);
    }
  };
  auto store_slice = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AQ; ++i) {
      const int q = tid + i * 256;
      *reinterpret_cast<u32x4*>(&As[buf][(q >> 2) * kPitch + (q & 3) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      const int q = tid + i * 256;
      *reinterpret_cast<u32x4*>(&Bs[buf][(q >> 2) * kPitch + (q & 3) * 8]) = rb[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = p.K / kBK;
  load_slice(0);
  store_slice(0);
  __syncthreads();
  const int lr = lane & 31;
  const int lk = (lane >> 5) * 8;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_slice((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      V8 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const V8*>(&As[buf][(wm * WTM + i * 32 + lr) * kPitch + kk + lk]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = *reinterpret_cast<const V8*>(&Bs[buf][(wn * WTN + j * 32 + lr) * kPitch + kk + lk]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Lowp<T>::mfma32(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_slice(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: bias, residual, ReLU, store.
  const float* bias = p.bias ? p.bias + (int64_t)g * p.bias_gstride : nullptr;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * WTN + j * 32 + lr;
    if (n >= p.N) continue;
    const float bn = bias ? bias[n] : 0.f;
    const int64_t ncol = (int64_t)(n >> 3) * p.c_nstride8 + (n & 7) + (int64_t)g * p.c_gstride;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m >= p.M) continue;
        const int64_t addr = (int64_t)m * p.ldc + ncol;
        float x = acc[i][j][v] + bn;
        if (p.R) x += p.r_f32 ? reinterpret_cast<const float*>(p.R)[addr]
                              : Lowp<T>::to_f32(reinterpret_cast<const T*>(p.R)[addr]);
        if (p.relu) x = x > 0.f ? x : 0.f;
        if (p.out_f32)
          reinterpret_cast<float*>(p.C)[addr] = x;
        else
          reinterpret_cast<T*>(p.C)[addr] = Lowp<T>::from_f32(x);
      }
    }
  }
}

template <typename T>
static hipError_t launch_gemm_t(const GemmParams& p, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, 2, 2>), dim3(tiles, p.groups), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, int lowp, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  return lowp == 0 ? launch_gemm_t<f16>(p, st) : launch_gemm_t<bf16>(p, st);
}

// ------------------------------------------------------------------ DLRM output layer (A4)
// One wave per candidate: z = w . h + b with fp32 accumulation in a fixed lane order and a
// fixed butterfly reduction (deterministic), then the fp32 sigmoid (CTR article, section 三:
// the prediction is returned in FP32).
template <typename T>
__global__ __launch_bounds__(256) void dlrm_output_kernel(const T* __restrict__ H, int M, int K,
                                                          const T* __restrict__ w, const float* __restrict__ b,
                                                          float* __restrict__ logits, float* __restrict__ out) {
  typedef typename Lowp<T>::vec8 V8;
  const int row = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const T* h = H + (int64_t)row * K;
  float acc = 0.f;
  for (int k = lane * 8; k < K; k += 512) {
    const V8 hv = load8(h + k);
    const V8 wv = load8(w + k);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += Lowp<T>::to_f32(hv[e]) * Lowp<T>::to_f32(wv[e]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) {
    const float z = acc + b[0];
    if (logits) logits[row] = z;
    out[row] = sigmoid_f32(z);
  }
}

hipError_t launch_dlrm_output(const void* H, int32_t M, int32_t K, const void* w, const float* b,
                              float* logits, float* out, int lowp, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int blocks = (M + 3) / 4;
  if (lowp == 0)
    hipLaunchKernelGGL(dlrm_output_kernel<f16>, dim3(blocks), dim3(256), 0, st, (const f16*)H, M, K,
                       (const f16*)w, b, logits, out);
  else
    hipLaunchKernelGGL(dlrm_output_kernel<bf16>, dim3(blocks), dim3(256), 0, st, (const bf16*)H, M, K,
                       (const bf16*)w, b, logits, out);
  return hipGetLastError();
}

}  // namespace cvr
