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
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace cvr {

// BM x BN block tile, WGM x WGN waves (4 in all), each wave an (BM/WGM) x (BN/WGN) tile of
// 32x32 MFMA sub-tiles; K advances in slices of kBK staged through LDS.  MFMA fragments of
// the next 16-wide k step are loaded before the current step's matrix instructions issue,
// so LDS latency overlaps them.  A-segment boundaries fall on slice boundaries, so each
// slice reads one segment: per-thread row pointers are rebuilt only when the loop enters a
// new segment (the row map is read there, not in the steady state).  AF32 selects fp32 A
// sources, rounded to the low-precision type as they are loaded.
template <typename T, int BM, int BN, int WGM, int WGN, bool AF32, int kBK = 32>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams p) {
  typedef typename Lowp<T>::vec8 V8;
  typedef typename std::conditional<AF32, float, T>::type AT;
  // LDS row layout.  64-wide slices: rows padded to 144 bytes, so both the 16-byte staging
  // writes (8 lanes fill one row) and the fragment reads (8 lanes read 8 rows) hit distinct
  // banks.  32-wide slices: unpadded 64-byte rows with the 16-byte chunk index XOR-ed with
  // (row/2)%4, which keeps the writes (8 lanes fill two rows) and the reads conflict-free.
  constexpr bool kSwz = kBK == 32;
  constexpr int kPitch = kSwz ? kBK : kBK + 8;
  constexpr int KC = kBK / 8;      // 16-byte (8-element) chunks per row of a slice
  constexpr int WTM = BM / WGM;
  constexpr int WTN = BN / WGN;
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int AQ = BM * KC / 256;  // A chunks per thread per slice
  constexpr int BQ = BN * KC / 256;
  static_assert(WGM * WGN == 4, "4 waves");
  static_assert(AQ >= 1 && BQ >= 1, "tile too small");

  // One LDS array: two A slices, two B slices; reused after the K loop to stage the output.
  constexpr int kSmemElems = 2 * BM * kPitch + 2 * BN * kPitch;
  __shared__ __align__(16) T smem[kSmemElems];
  auto As = [&](int buf) { return smem + buf * (BM * kPitch); };
  auto Bs = [&](int buf) { return smem + 2 * BM * kPitch + buf * (BN * kPitch); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN;
  const int wn = wave % WGN;
  const int g = blockIdx.y;

  // XCD-aware renumbering: hardware dispatch puts block b on XCD b % 8; tiles that share an
  // A row-block (consecutive in N) land on one XCD and reuse it from its L2.
  const int ntn = (p.N + BN - 1) / BN;
  const int total = gridDim.x;
  int lb = blockIdx.x;
  if ((total & 7) == 0) lb = (lb & 7) * (total >> 3) + (lb >> 3);
  const int m0 = (lb / ntn) * BM;
  const int n0 = (lb % ntn) * BN;

  // Per-thread chunk coordinates (fixed for the whole K loop).
  const int cq = tid % KC;  // chunk within a slice row (the same for every i below since 256 % KC == 0)
  int am[AQ];
#pragma unroll
  for (int i = 0; i < AQ; ++i) {
    const int m = m0 + (tid + i * 256) / KC;
    am[i] = m < p.M ? m : p.M - 1;
  }
  const T* wptr[BQ];
#pragma unroll
  for (int i = 0; i < BQ; ++i) {
    int n = n0 + (tid + i * 256) / KC;
    n = n < p.N ? n : p.N - 1;
    wptr[i] = reinterpret_cast<const T*>(p.W) + (int64_t)g * p.w_gstride + (int64_t)n * p.K + cq * 8;
  }

  // Segment state: row pointers of the current segment (chunk cq of each row at col0).
  int seg = -1, seg_kb = 0, seg_end = 0;
  int64_t seg_kstride = 8;
  const AT* aptr[AQ];
  auto enter_segment = [&](int k0) {
    while (k0 >= seg_end) {
      ++seg;
      seg_kb = seg == 0 ? 0 : p.seg[seg - 1].k_end;
      seg_end = p.seg[seg].k_end;
    }
    const ASeg& S = p.seg[seg];
    seg_kstride = S.kstride8;
#pragma unroll
    for (int i = 0; i < AQ; ++i) {
      const int64_t row = S.rowmap ? (int64_t)S.rowmap[am[i]] : (int64_t)am[i];
      aptr[i] = reinterpret_cast<const AT*>(S.ptr) + (int64_t)g * S.gstride + row * S.ld +
                (int64_t)((S.col0 >> 3) + cq) * S.kstride8;
    }
  };

  // Two register staging sets: the slice two steps ahead is in flight while the next one
  // waits in registers for its turn in LDS, so each global load has two slices of MFMA work
  // to complete.
  u32x4 ra[2][AQ], rb[2][BQ];
  auto load_slice = [&](int k0, int set) {
    if (k0 >= seg_end) enter_segment(k0);
    const int64_t off = (int64_t)((k0 - seg_kb) >> 3) * seg_kstride;
#pragma unroll
    for (int i = 0; i < AQ; ++i) {
      if constexpr (AF32) {
        const float4* src = reinterpret_cast<const float4*>(aptr[i] + off);
        const float4 x0 = src[0], x1 = src[1];
        V8 v;
        v[0] = Lowp<T>::from_f32(x0.x); v[1] = Lowp<T>::from_f32(x0.y);
        v[2] = Lowp<T>::from_f32(x0.z); v[3] = Lowp<T>::from_f32(x0.w);
        v[4] = Lowp<T>::from_f32(x1.x); v[5] = Lowp<T>::from_f32(x1.y);
        v[6] = Lowp<T>::from_f32(x1.z); v[7] = Lowp<T>::from_f32(x1.w);
        ra[set][i] = *reinterpret_cast<const u32x4*>(&v);
      } else {
        ra[set][i] = *reinterpret_cast<const u32x4*>(aptr[i] + off);
      }
    }
#pragma unroll
    for (int i = 0; i < BQ; ++i) rb[set][i] = *reinterpret_cast<const u32x4*>(wptr[i] + k0);
  };
  auto store_slice = [&](int buf, int set) {
#pragma unroll
    for (int i = 0; i < AQ; ++i) {
      const int q = tid + i * 256;
      const int r = q / KC;
      const int c = kSwz ? ((q % KC) ^ ((r >> 1) & 3)) : (q % KC);
      *reinterpret_cast<u32x4*>(As(buf) + r * kPitch + c * 8) = ra[set][i];
    }
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      const int q = tid + i * 256;
      const int r = q / KC;
      const int c = kSwz ? ((q % KC) ^ ((r >> 1) & 3)) : (q % KC);
      *reinterpret_cast<u32x4*>(Bs(buf) + r * kPitch + c * 8) = rb[set][i];
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
  const int lr = lane & 31;
  const int lc = lane >> 5;                       // which 8-element half of a 16-wide k step
  const int sw = kSwz ? ((lr >> 1) & 3) : 0;      // row swizzle (rows differ by multiples of 8 across sub-tiles)
  const int arow = (wm * WTM + lr) * kPitch;
  const int brow = (wn * WTN + lr) * kPitch;
  auto koff = [&](int ks) { return ((ks * 2 + lc) ^ sw) * 8; };  // element offset of this lane's chunk at k step ks

  // MFMAs of one K step on LDS buffer kt&1.
  auto compute = [&](int kt) {
    const T* Ab = As(kt & 1);
    const T* Bb = Bs(kt & 1);
    V8 a[2][FM], b[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a[0][i] = *reinterpret_cast<const V8*>(Ab + arow + i * 32 * kPitch + koff(0));
#pragma unroll
    for (int j = 0; j < FN; ++j) b[0][j] = *reinterpret_cast<const V8*>(Bb + brow + j * 32 * kPitch + koff(0));
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kBK / 16) {
#pragma unroll
        for (int i = 0; i < FM; ++i) a[cur ^ 1][i] = *reinterpret_cast<const V8*>(Ab + arow + i * 32 * kPitch + koff(ks + 1));
#pragma unroll
        for (int j = 0; j < FN; ++j) b[cur ^ 1][j] = *reinterpret_cast<const V8*>(Bb + brow + j * 32 * kPitch + koff(ks + 1));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Lowp<T>::mfma32(a[cur][i], b[cur][j], acc[i][j]);
    }
  };
  // One pipelined step: slice kt+2 (clamped to the last slice) loads into register set SET —
  // a compile-time index and an unconditional load, so the loads stay in flight and the
  // wait before the LDS store covers only the older set — while MFMAs run on buffer kt&1;
  // then slice kt+1 moves from the other set into the other buffer.  Past the last slice the
  // loads repeat it and land in a buffer that is not read again.
  auto step = [&](int kt, auto set_c) {
    constexpr int SET = decltype(set_c)::value;
    load_slice((kt + 2 < nk ? kt + 2 : nk - 1) * kBK, SET);
    compute(kt);
    store_slice((kt & 1) ^ 1, SET ^ 1);
    __syncthreads();
  };

  load_slice(0, 0);
  load_slice((nk > 1 ? 1 : 0) * kBK, 1);
  store_slice(0, 0);
  __syncthreads();
  int kt = 0;
#pragma unroll 1
  for (; kt + 2 <= nk; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < nk) compute(kt);
  __syncthreads();

  const float* bias = p.bias ? p.bias + (int64_t)g * p.bias_gstride : nullptr;
  constexpr bool kCanStageF32 = 4 * 32 * (WTN + 8) * 4 <= kSmemElems * (int)sizeof(T);
  constexpr bool kCanStageLp = 4 * 32 * (WTN + 8) * (int)sizeof(T) <= kSmemElems * (int)sizeof(T);
  if ((p.out_f32 ? kCanStageF32 : kCanStageLp) && p.c_nstride8 == 8 && !p.R && (p.ldc & 7) == 0) {
    // Contiguous output rows: stage each wave's tile 32 rows at a time through LDS (free after
    // the K loop) and write it back as 16-byte row segments.  Every thread runs the same number
    // of rounds, so the block barriers below are uniform.
    constexpr int OP = WTN + 8;  // staged row pitch in 4-byte words (fp32) or elements (lowp)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (p.out_f32) {
        float* st = reinterpret_cast<float*>(smem) + wave * 32 * OP;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int nl = j * 32 + lr;
          const int n = n0 + wn * WTN + nl;
          const float bn = (bias && n < p.N) ? bias[n] : 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float x = acc[i][j][v] + bn;
            if (p.relu) x = x > 0.f ? x : 0.f;
            st[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * OP + nl] = x;
          }
        }
        __syncthreads();
        constexpr int CPR = WTN / 4;
#pragma unroll
        for (int c = lane; c < 32 * CPR; c += 64) {
          const int rl = c / CPR, cc = c % CPR;
          const int m = m0 + wm * WTM + i * 32 + rl;
          const int n = n0 + wn * WTN + cc * 4;
          if (m < p.M && n < p.N) {
            const float4 v = *reinterpret_cast<const float4*>(&st[rl * OP + cc * 4]);
            float* dst = reinterpret_cast<float*>(p.C) + (int64_t)g * p.c_gstride + (int64_t)m * p.ldc + n;
            if (n + 4 <= p.N) {
              *reinterpret_cast<float4*>(dst) = v;
            } else {
              const int cnt = p.N - n;
              dst[0] = v.x;
              if (cnt > 1) dst[1] = v.y;
              if (cnt > 2) dst[2] = v.z;
            }
          }
        }
      } else {
        T* st = smem + wave * 32 * OP;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int nl = j * 32 + lr;
          const int n = n0 + wn * WTN + nl;
          const float bn = (bias && n < p.N) ? bias[n] : 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float x = acc[i][j][v] + bn;
            if (p.relu) x = x > 0.f ? x : 0.f;
            st[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * OP + nl] = Lowp<T>::from_f32(x);
          }
        }
        __syncthreads();
        constexpr int CPR = WTN / 8;
#pragma unroll
        for (int c = lane; c < 32 * CPR; c += 64) {
          const int rl = c / CPR, cc = c % CPR;
          const int m = m0 + wm * WTM + i * 32 + rl;
          const int n = n0 + wn * WTN + cc * 8;
          if (m < p.M && n < p.N) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(&st[rl * OP + cc * 8]);
            T* dst = reinterpret_cast<T*>(p.C) + (int64_t)g * p.c_gstride + (int64_t)m * p.ldc + n;
            if (n + 8 <= p.N) {
              *reinterpret_cast<u32x4*>(dst) = v;
            } else {
              const int cnt = p.N - n;
              typename Lowp<T>::vec8 t = *reinterpret_cast<const typename Lowp<T>::vec8*>(&v);
#pragma unroll
              for (int e = 0; e < 7; ++e)
                if (e < cnt) dst[e] = t[e];
            }
          }
        }
      }
      __syncthreads();
    }
    return;
  }

  // General epilogue (strided output layouts, residual): bias, residual, ReLU, store.
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

// Tile choice (measured on the 1024x1024 hidden layers): 256x256 with 32-wide slices when
// the grid holds at least four tiles per CU; otherwise 128x128 (64-wide slices when every
// K-segment boundary allows, else 32-wide); 64x64 when even 128x128 cannot cover the chip
// (the per-candidate GEMMs of the CVR model at small batch).
template <typename T, bool AF32>
static hipError_t launch_gemm_t(const GemmParams& p, hipStream_t st) {
  auto tiles = [&](int bm, int bn) { return ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn); };
  bool bk64 = p.K % 64 == 0;
  for (int s = 0; s < p.nseg; ++s) bk64 = bk64 && p.seg[s].k_end % 64 == 0;
  const char* env = getenv("CVR_GEMM_TILE");
  int tile = env ? atoi(env) : 0;
  if (!tile) {
    if (p.N % 256 == 0 && (int64_t)tiles(256, 256) * p.groups >= 1024) tile = 256;
    else if ((int64_t)tiles(128, 128) * p.groups >= 256) tile = 128;
    else tile = 64;
  }
  const dim3 blk(256);
  if (tile == 256) {
    hipLaunchKernelGGL((gemm_kernel<T, 256, 256, 2, 2, AF32, 32>), dim3(tiles(256, 256), p.groups), blk, 0, st, p);
  } else if (tile == 128) {
    if (bk64) hipLaunchKernelGGL((gemm_kernel<T, 128, 128, 2, 2, AF32, 64>), dim3(tiles(128, 128), p.groups), blk, 0, st, p);
    else hipLaunchKernelGGL((gemm_kernel<T, 128, 128, 2, 2, AF32, 32>), dim3(tiles(128, 128), p.groups), blk, 0, st, p);
  } else {
    if (bk64) hipLaunchKernelGGL((gemm_kernel<T, 64, 64, 2, 2, AF32, 64>), dim3(tiles(64, 64), p.groups), blk, 0, st, p);
    else hipLaunchKernelGGL((gemm_kernel<T, 64, 64, 2, 2, AF32, 32>), dim3(tiles(64, 64), p.groups), blk, 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, int lowp, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.K % 32) return hipErrorInvalidValue;
  int kb = 0;
  for (int s = 0; s < p.nseg; ++s) {
    if (p.seg[s].k_end % 32 || p.seg[s].col0 % 8 || p.seg[s].k_end <= kb || p.seg[s].f32 != p.seg[0].f32)
      return hipErrorInvalidValue;
    kb = p.seg[s].k_end;
  }
  if (kb != p.K) return hipErrorInvalidValue;
  const bool f32 = p.seg[0].f32 != 0;
  if (lowp == 0) return f32 ? launch_gemm_t<f16, true>(p, st) : launch_gemm_t<f16, false>(p, st);
  return f32 ? launch_gemm_t<bf16, true>(p, st) : launch_gemm_t<bf16, false>(p, st);
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
