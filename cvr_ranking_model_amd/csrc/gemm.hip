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
// sources, rounded to the low-precision type as they move from registers to LDS.
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

  // NSET register staging sets: the slices up to NSET steps ahead are in flight while the next
  // one waits in registers for its turn in LDS, so each global load has NSET slices of MFMA
  // work to complete.  Three sets for the small tiles, whose short slices (and few waves per
  // CU) leave the loads too little time otherwise (C3, 512 samples: step -2.5%); two for
  // 128 x 128, where a third set costs occupancy and gained nothing.  An fp32 A chunk stays
  // fp32 in its set (rf) and is rounded on its way to LDS: rounding at the load would wait for
  // the load there.
  constexpr int NSET = BM * BN <= 64 * 128 ? 3 : 2;
  u32x4 ra[NSET][AQ], rb[NSET][BQ];
  f32x4 rf[NSET][AQ][2];
  auto load_slice = [&](int k0, int set) {
    if (k0 >= seg_end) enter_segment(k0);
    const int64_t off = (int64_t)((k0 - seg_kb) >> 3) * seg_kstride;
#pragma unroll
    for (int i = 0; i < AQ; ++i) {
      if constexpr (AF32) {
        const f32x4* src = reinterpret_cast<const f32x4*>(aptr[i] + off);
        rf[set][i][0] = src[0];
        rf[set][i][1] = src[1];
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
      if constexpr (AF32) {
        V8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = Lowp<T>::from_f32(rf[set][i][0][e]);
          v[4 + e] = Lowp<T>::from_f32(rf[set][i][1][e]);
        }
        *reinterpret_cast<V8*>(As(buf) + r * kPitch + c * 8) = v;
      } else {
        *reinterpret_cast<u32x4*>(As(buf) + r * kPitch + c * 8) = ra[set][i];
      }
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
  // One pipelined step: slice kt+NSET (clamped to the last slice) loads into register set
  // SET = kt % NSET -- a compile-time index and an unconditional load, so the loads stay in
  // flight and the wait before the LDS store covers only the oldest set -- while MFMAs run on
  // buffer kt&1; then slice kt+1 moves from its set into the other buffer.  Past the last slice
  // the loads repeat it and land in a buffer that is not read again.
  auto step = [&](int kt, auto set_c) {
    constexpr int SET = decltype(set_c)::value;
    load_slice((kt + NSET < nk ? kt + NSET : nk - 1) * kBK, SET);
    compute(kt);
    store_slice((kt & 1) ^ 1, (SET + 1) % NSET);
    __syncthreads();
  };
  auto steps = [&](int kt, auto count_c) {  // steps kt .. kt+count-1, kt a multiple of NSET
#pragma unroll
    for (int j = 0; j < NSET; ++j)
      if (j < decltype(count_c)::value) {
        if (j == 0) step(kt, std::integral_constant<int, 0>{});
        if (j == 1) step(kt + 1, std::integral_constant<int, 1>{});
        if (j == 2) step(kt + 2, std::integral_constant<int, 2 % NSET>{});
      }
  };

#pragma unroll
  for (int j = 0; j < NSET; ++j) load_slice((j < nk ? j : nk - 1) * kBK, j);
  store_slice(0, 0);
  __syncthreads();
  int kt = 0;
#pragma unroll 1
  for (; kt + NSET < nk; kt += NSET) steps(kt, std::integral_constant<int, NSET>{});
  // the last 1..NSET slices: a step for each but the last, which only computes
  if (nk - kt == 2) steps(kt, std::integral_constant<int, 1>{});
  if (NSET == 3 && nk - kt == 3) steps(kt, std::integral_constant<int, 2>{});
  compute(nk - 1);
  __syncthreads();

  const float* bias = p.bias ? p.bias + (int64_t)g * p.bias_gstride : nullptr;
  constexpr bool kCanStageF32 = 4 * 32 * (WTN + 8) * 4 <= kSmemElems * (int)sizeof(T);
  constexpr bool kCanStageLp = 4 * 32 * (WTN + 8) * (int)sizeof(T) <= kSmemElems * (int)sizeof(T);
  // An fp32 residual is added on the way out of the staging area for fp32 outputs (no ReLU may
  // follow it there), and before the ReLU on the way in for low-precision outputs.
  const bool stage_r = !p.R || (p.r_f32 && (p.out_f32 ? (!p.relu && (!p.r_rowmap || (p.r_ld & 3) == 0)) : true));
  if ((p.out_f32 ? kCanStageF32 : kCanStageLp) && p.c_nstride8 == 8 && stage_r && (p.ldc & 7) == 0) {
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
            if (p.relu && (p.relu_end == 0 || n < p.relu_end)) x = relu_f32(x);
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
            float4 v = *reinterpret_cast<const float4*>(&st[rl * OP + cc * 4]);
            const int64_t off = (int64_t)g * p.c_gstride + (int64_t)m * p.ldc + n;
            float* dst = reinterpret_cast<float*>(p.C) + off;
            const float* res = p.R ? reinterpret_cast<const float*>(p.R) +
                                         (p.r_rowmap ? (int64_t)p.r_rowmap[m] * p.r_ld + n : off)
                                   : nullptr;
            if (n + 4 <= p.N) {
              if (res) {
                const float4 r4 = *reinterpret_cast<const float4*>(res);
                v.x += r4.x;
                v.y += r4.y;
                v.z += r4.z;
                v.w += r4.w;
              }
              *reinterpret_cast<float4*>(dst) = v;
              if (p.C2) {
                typedef T T4 __attribute__((ext_vector_type(4)));
                T4 vb;
                vb[0] = Lowp<T>::from_f32(v.x);
                vb[1] = Lowp<T>::from_f32(v.y);
                vb[2] = Lowp<T>::from_f32(v.z);
                vb[3] = Lowp<T>::from_f32(v.w);
                *reinterpret_cast<T4*>(reinterpret_cast<T*>(p.C2) + (int64_t)m * p.ldc2 + n) = vb;
              }
            } else {
              const int cnt = p.N - n;
              const float vv[3] = {v.x, v.y, v.z};
#pragma unroll
              for (int e = 0; e < 3; ++e)
                if (e < cnt) {
                  const float x = res ? vv[e] + res[e] : vv[e];
                  dst[e] = x;
                  if (p.C2) reinterpret_cast<T*>(p.C2)[(int64_t)m * p.ldc2 + n + e] = Lowp<T>::from_f32(x);
                }
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
            if (p.R) {
              const int m = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
              if (m < p.M && n < p.N)
                x += reinterpret_cast<const float*>(p.R)[p.r_rowmap ? (int64_t)p.r_rowmap[m] * p.r_ld + n
                                                                    : (int64_t)g * p.c_gstride + (int64_t)m * p.ldc + n];
            }
            if (p.relu && (p.relu_end == 0 || n < p.relu_end)) x = relu_f32(x);
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
        const int64_t raddr = p.r_rowmap ? (int64_t)p.r_rowmap[m] * p.r_ld + ncol : addr;
        float x = acc[i][j][v] + bn;
        if (p.R) x += p.r_f32 ? reinterpret_cast<const float*>(p.R)[raddr]
                              : Lowp<T>::to_f32(reinterpret_cast<const T*>(p.R)[raddr]);
        if (p.relu && (p.relu_end == 0 || n < p.relu_end)) x = relu_f32(x);
        if (p.out_f32) {
          reinterpret_cast<float*>(p.C)[addr] = x;
          if (p.C2) reinterpret_cast<T*>(p.C2)[(int64_t)m * p.ldc2 + n] = Lowp<T>::from_f32(x);
        } else {
          reinterpret_cast<T*>(p.C)[addr] = Lowp<T>::from_f32(x);
        }
      }
    }
  }
}

// Hardware dispatch puts block b on XCD b % 8, in order b / 8 within it.  Renumber blocks so
// each XCD receives one contiguous run of logical tiles (a bijection for any block count):
// the tiles that share an A row-block (consecutive in N) then run together on one XCD and
// reuse it from that XCD's L2.
__device__ __forceinline__ int xcd_tile(int b, int total) {
  const int q = total >> 3, rem = total & 7, x = b & 7;
  return x * q + (x < rem ? x : rem) + (b >> 3);
}

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 s_waitcnt
// encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte global -> LDS transfer per lane, written to lds_wave_base + 16 * lane (the LDS
// base must be the same for every lane of the wave).
__device__ __forceinline__ void load_lds16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Wide-layer GEMM, persistent: each block walks a list of BM x BN output tiles (256 x 256 with
// 8 waves, one block per CU; or 256 x 128 with 4 waves, two blocks per CU), every wave a
// 128 x 64 tile of MFMA 32x32x16 (two waves per SIMD either way).  K advances in BK-wide
// slices (32 or 64) that go from global memory straight into an NS-slot LDS ring (no register
// staging), and the slice stream runs across tile boundaries: slice s+NS is requested as soon
// as slot s%NS is released, mid-way through slice s, so the next tile's first slices are in
// flight while this tile's epilogue runs.  Transfers and fragment reads are interleaved with
// the matrix instructions so that their issue hides behind the MFMA pipe.
// Stores and loads share one vector-memory counter, so a store holds up every later wait.
// The epilogue therefore first lets the in-flight slices land and only then issues its stores;
// the next tile's first NS-1 slices need no wait, and the first wait that does come (for slice
// NS, requested after the stores) is two slices of matrix work later.
// LDS banks: a 16-byte read is served 16 lanes (256 bytes) at a time, and the 16 lanes of a
// fragment read cover 16 consecutive rows at one k chunk.  Rows are BK*2 bytes with the chunk
// index XOR-ed with swz(row) = (row/4)%4 for 64-byte rows and (row/2)%8 for 128-byte rows,
// which places those 16 reads on 16 distinct 16-byte bank groups.  The loaders choose which
// chunk each lane fetches so that the fixed lane->LDS placement of a transfer (lane l at byte
// 16 l) realises the layout.  Everything lives in one LDS allocation (ring, per-wave output
// staging, bias): the waits on the ring are the explicit ones below.
// The W fragment is the MFMA's first operand, so each lane's accumulators hold 4 consecutive
// output columns of one row; the epilogue stages them through a per-wave LDS area and writes
// whole row segments.
// Tile order: each XCD gets one contiguous run of tiles and its blocks take them round-robin,
// so tiles that share an A row-block run at the same time on the same L2.
// Requirements (checked by the launcher): N % BN == 0, N <= kBigMaxN, K and every A-segment
// boundary multiples of BK, 16-bit A sources and output, contiguous output rows with
// ldc % 8 == 0, no residual, a grid that is a multiple of 8 blocks.
constexpr int kBigMaxN = 1024;
template <typename T, int BM, int BN, int BK, int NS, int MINB>
__global__ __launch_bounds__(BN / 64 * 128, MINB) void gemm_big_kernel(const GemmParams p) {
  typedef typename Lowp<T>::vec8 V8;
  constexpr int KC = BK / 8;              // 16-byte chunks per slice row
  constexpr int RPI = 64 / KC;            // rows filled by one wave transfer (1 KB)
  constexpr int NW = BN / 64 * 2;         // waves: 2 along M x BN/64 along N, each 128 x 64
  constexpr int NT = NW * 64;
  constexpr int TPA = BM / RPI / NW;      // transfers per wave per slice: A rows
  constexpr int TPB = BN / RPI / NW;      //                                W rows
  constexpr int L = TPA + TPB;
  constexpr int KS = BK / 16;             // MFMA k steps per slice
  constexpr int WTM = 128, WTN = 64;       // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int kSlot = (BM + BN) * BK;   // elements per ring slot: BM A rows, then BN W rows
  constexpr int kStagePitch = WTN * 2 + 16;  // bytes per staged output row (odd multiple of 16)
  constexpr int RPS = 1024 / (WTN * 2);      // staged rows written back per wave instruction
  constexpr int LPR = WTN / 8;               // lanes per staged row on the way out (16 bytes each)
  static_assert(BK == 32 || BK == 64, "slice width");
  static_assert(BM == 256, "two 128-row wave tiles along M");
  static_assert(TPA >= 1 && TPB >= 1 && BM % (NW * RPI) == 0 && BN % (NW * RPI) == 0, "loader shape");
  static_assert(NS >= 2 && L * (NS - 2) < 64, "ring depth");
  // One LDS allocation: the ring, the per-wave staging areas, the bias of all N columns and the
  // output-layer weights of all N columns (fused output layer only).
  constexpr int kRingBytes = NS * kSlot * (int)sizeof(T);
  // Staged output rows per pass: a whole 32-row m-tile, or half of it when the ring leaves too
  // little LDS.
  constexpr int SR = kRingBytes + NW * 32 * kStagePitch + 2 * kBigMaxN * 4 <= 160 * 1024 ? 32 : 16;
  constexpr int kStageBytes = NW * SR * kStagePitch;
  __shared__ __align__(1024) char lds[kRingBytes + kStageBytes + 2 * kBigMaxN * 4];
  T* const smem = reinterpret_cast<T*>(lds);
  char* const stage = lds + kRingBytes + (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * SR * kStagePitch;
  float* const bias_s = reinterpret_cast<float*>(lds + kRingBytes + kStageBytes);
  float* const ow_s = bias_s + kBigMaxN;
  static_assert(WTN == kOutGroup, "one output-layer partial per wave column group");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);
  const int g = blockIdx.y;
  const int ntn = p.N / BN;
  const int total = ((p.M + BM - 1) / BM) * ntn;
  const int x = blockIdx.x & 7, stride = gridDim.x >> 3;
  const int tq = total >> 3, trem = total & 7;
  const int first = x * tq + (x < trem ? x : trem) + (blockIdx.x >> 3);
  const int last = (x + 1) * tq + (x + 1 < trem ? x + 1 : trem);
  if (first >= last) return;
  for (int c = tid; c < p.N; c += NT) bias_s[c] = p.bias ? p.bias[(int64_t)g * p.bias_gstride + c] : 0.f;
  if (p.ow)
    for (int c = tid; c < p.N; c += NT) ow_s[c] = Lowp<T>::to_f32(reinterpret_cast<const T*>(p.ow)[c]);

  auto swz = [](int row) { return KC == 4 ? (row >> 2) & 3 : (row >> 1) & 7; };
  // Loader: transfer (NW i + wave) fills rows RPI*(NW i+wave) .. +RPI-1; lane l lands in row
  // l/KC of them at slot l%KC and must fetch k-chunk slot ^ swz(row).  swz(row) is the same
  // for every i (RPI*NW is a multiple of the swizzle period), so each lane has one k-chunk.
  const int lrow = lane / KC;
  const int kch = (lane % KC) ^ swz(RPI * wave + lrow);
  const int nk = p.K / BK;

  // Issue cursor: tile it, slice ik (runs NS slices ahead of the compute cursor).
  int it = first, ik = 0;
  int am[TPA];
  const T* wrow[TPB];
  int seg = -1, seg_kb = 0, seg_end = 0;
  int64_t seg_kstride = 8;
  const T* aptr[TPA];
  auto set_tile = [&](int t) {
    const int tm0 = (t / ntn) * BM, tn0 = (t % ntn) * BN;
#pragma unroll
    for (int i = 0; i < TPA; ++i) {
      const int r = tm0 + RPI * (NW * i + wave) + lrow;
      am[i] = r < p.M ? r : p.M - 1;
    }
#pragma unroll
    for (int i = 0; i < TPB; ++i)
      wrow[i] = reinterpret_cast<const T*>(p.W) + (int64_t)g * p.w_gstride +
                (int64_t)(tn0 + RPI * (NW * i + wave) + lrow) * p.K + kch * 8;
    seg = -1;
    seg_kb = 0;
    seg_end = 0;
  };
  auto enter_segment = [&](int k0) {
    while (k0 >= seg_end) {
      ++seg;
      seg_kb = seg == 0 ? 0 : p.seg[seg - 1].k_end;
      seg_end = p.seg[seg].k_end;
    }
    const ASeg& S = p.seg[seg];
    seg_kstride = S.kstride8;
#pragma unroll
    for (int i = 0; i < TPA; ++i) {
      const int64_t row = S.rowmap ? (int64_t)S.rowmap[am[i]] : (int64_t)am[i];
      aptr[i] = reinterpret_cast<const T*>(S.ptr) + (int64_t)g * S.gstride + row * S.ld +
                (int64_t)((S.col0 >> 3) + kch) * S.kstride8;
    }
  };
  // Make the issue cursor's slice addressable (its A segment current).
  auto prepare = [&]() {
    if (ik * BK >= seg_end) enter_segment(ik * BK);
  };
  // Move the issue cursor on; past this block's last slice it stays there, so the remaining
  // requests repeat that slice into slots that are not read any more.
  auto advance = [&]() {
    if (ik + 1 < nk) {
      ++ik;
    } else if (it + stride < last) {
      it += stride;
      ik = 0;
      set_tile(it);
    }
  };
  auto issue = [&](int slot) {
    const int k0 = ik * BK;
    const int64_t off = (int64_t)((k0 - seg_kb) >> 3) * seg_kstride;
    T* sA = smem + slot * kSlot;
    T* sB = sA + BM * BK;
#pragma unroll
    for (int i = 0; i < TPA; ++i) load_lds16(aptr[i] + off, sA + (NW * i + wave) * 512);
#pragma unroll
    for (int i = 0; i < TPB; ++i) load_lds16(wrow[i] + k0, sB + (NW * i + wave) * 512);
  };

  const int lr = lane & 31, lc = lane >> 5;
  const int sw = swz(lr);
  const int arow = (wm * WTM + lr) * BK;
  const int brow = BM * BK + (wn * WTN + lr) * BK;
  auto read_frags = [&](int slot, int ks, V8 (&fa)[FM], V8 (&fb)[FN]) {
    const T* base = smem + slot * kSlot;
    const int c = ((2 * ks + lc) ^ sw) * 8;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const V8*>(base + arow + i * 32 * BK + c);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const V8*>(base + brow + j * 32 * BK + c);
  };
  f32x16 acc[FM][FN];
  auto mfmas = [&](const V8 (&fa)[FM], const V8 (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = Lowp<T>::mfma32(fb[j], fa[i], acc[i][j]);
  };
  constexpr int NMF = FM * FN;  // MFMAs per k step
  constexpr int NRD = FM + FN;  // fragment reads per k step

  // Every iteration requests exactly one slice, so exactly L * (NS - 2) transfers are younger
  // than slice s+1 when the loop waits for it.
  set_tile(it);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    prepare();
    issue(s);
    advance();
  }
  V8 fa[2][FM], fb[2][FN];
  wait_vmcnt<L * (NS - 1)>();
  __syncthreads();
  read_frags(0, 0, fa[0], fb[0]);
  int slot = 0;
  bool landed = false;  // the first NS-1 slices of this tile are known to be in LDS

#pragma unroll 1
  for (int tc = first; tc < last; tc += stride) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
      const int next = slot == NS - 1 ? 0 : slot + 1;
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks) {
        read_frags(slot, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        mfmas(fa[ks & 1], fb[ks & 1]);
#pragma unroll
        for (int q = 0; q < NRD; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, NMF / NRD > 0 ? NMF / NRD : 1, 0);  // MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              // 1 LDS read
        }
      }
      prepare();
      // Slice s+1 has landed for this wave (the barrier covers the other waves), and every
      // wave is done reading slot s%NS before it is refilled.
      if (!(landed && kt < NS - 1)) wait_vmcnt<L * (NS - 2)>();
      __syncthreads();
      issue(slot);
      read_frags(next, 0, fa[KS & 1], fb[KS & 1]);
      mfmas(fa[(KS - 1) & 1], fb[(KS - 1) & 1]);
      // next slice's first fragments early (they gate the next iteration), transfers after
#pragma unroll
      for (int q = 0; q < NRD; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      }
#pragma unroll
      for (int q = 0; q < L; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 transfer
      }
      advance();
      slot = next;
    }

    // Epilogue: lane holds, for m-tile i and n-tile j, row m = .. + lane%32 and the four
    // consecutive columns n = .. + 8*q + 4*(lane/32) + 0..3 for q = 0..3.  Per m-tile the wave
    // writes its 32 x WTN block into its own staging area (8-byte writes; a pitch that is an
    // odd multiple of 8 bytes keeps 32 rows on distinct banks) and reads it back as rows.
    const int m0 = (tc / ntn) * BM, ncol0 = (tc % ntn) * BN + wn * WTN;
    if (p.ow) {
      // Fused output layer: per row, the rounded activations of this wave's WTN columns times
      // the output weights, in a fixed order: a lane half holds every other 4-column run (the
      // lower half the runs starting at 8r, the upper half those at 8r + 4); each half sums its
      // runs in column order, every run a fused multiply-add chain over its 4 columns, and the
      // row's partial is the lower half's sum plus the upper half's.  Nothing of C is stored.
      float dot[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) dot[i] = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = ncol0 + j * 32 + 8 * q + 4 * lc;
          const float4 b4 = *reinterpret_cast<const float4*>(&bias_s[col]);
          const float4 w4 = *reinterpret_cast<const float4*>(&ow_s[col]);
          const float bq[4] = {b4.x, b4.y, b4.z, b4.w}, wq[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            float run = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = acc[i][j][4 * q + e] + bq[e];
              if (p.relu) v = relu_f32(v);
              run = fmaf(Lowp<T>::to_f32(Lowp<T>::from_f32(v)), wq[e], run);
            }
            dot[i] += run;
          }
        }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const float upper = __shfl_xor(dot[i], 32);  // lanes 0-31 receive the upper half's sums
        dot[i] += upper;
      }
      wait_vmcnt<0>();  // the next tile's first slices land before any store
      if (lc == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int m = m0 + wm * WTM + i * 32 + lr;
          if (m < p.M) p.opart[(int64_t)(ncol0 / kOutGroup) * p.opart_ld + m] = dot[i];
        }
      }
      landed = true;
      continue;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int mrow0 = m0 + wm * WTM + i * 32;
      typedef T T4 __attribute__((ext_vector_type(4)));
      T4 o[FN][4];
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = j * 32 + 8 * q + 4 * lc;
          const float4 b4 = *reinterpret_cast<const float4*>(&bias_s[ncol0 + col]);
          const float bq[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v = acc[i][j][4 * q + e] + bq[e];
            if (p.relu) v = relu_f32(v);
            o[j][q][e] = Lowp<T>::from_f32(v);
          }
        }
#pragma unroll
      for (int h = 0; h < 32 / SR; ++h) {
        if (SR == 32 || (lr >> 4) == h) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<T4*>(stage + (lr - h * SR) * kStagePitch + (j * 32 + 8 * q + 4 * lc) * 2) = o[j][q];
        }
        if (i == 0 && h == 0) wait_vmcnt<0>();  // the next tile's first slices land before any store
#pragma unroll
        for (int rr = 0; rr < SR / RPS; ++rr) {
          const int r = rr * RPS + lane / LPR;
          const uint4 v = *reinterpret_cast<const uint4*>(stage + r * kStagePitch + (lane % LPR) * 16);
          const int m = mrow0 + h * SR + r;
          if (m < p.M)
            *reinterpret_cast<uint4*>(reinterpret_cast<T*>(p.C) + (int64_t)g * p.c_gstride + (int64_t)m * p.ldc +
                                      ncol0 + 8 * (lane % LPR)) = v;
        }
      }
    }
    landed = true;
  }
  // Requests past the last slice must land before the block's LDS is released.
  wait_vmcnt<0>();
}

// Persistent grid for the wide-layer kernel: per_cu blocks per CU, a multiple of 8 (every XCD
// gets the same number of blocks), never more than the tiles need.
static int big_grid(int tiles, int per_cu) {
  static int cus = 0;
  if (!cus) {
    int dev = 0, n = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    cus = n;
  }
  int b = cus * per_cu < tiles ? cus * per_cu : tiles;
  b = (b + 7) & ~7;
  return b < 8 ? 8 : b;
}

// Tile choice: the persistent wide-layer kernel when its layout requirements hold and there is
// at least a tile per CU (256 x 256 tiles when N allows, else 256 x 128); otherwise 128x128
// (64-wide slices when every K-segment boundary allows, else 32-wide) when its tiles keep at
// least three quarters of the CUs busy (measured: the CVR expert GEMM, 224 tiles of K = 2048,
// runs 36 us against 58 us as 64x64); below that 64x128 when the caller asks for a group's
// whole width (N <= 128) in one tile (the CVR query GEMM at 500 candidates per request: 23 us
// against 33 us as 64x64, whose six tiles per row block re-read its 1,792 fp32 A columns; at
// one candidate per request the 64x64 grid's wider spread is faster), else 64x64 (the
// per-candidate GEMMs of the CVR model at small batch).
static int choose_tile(const GemmParams& p, bool af32) {
  auto tiles = [&](int bm, int bn) { return ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn); };
  int tile = 0;
  const bool big_ok = !af32 && !p.out_f32 && p.N % 128 == 0 && p.N <= kBigMaxN && p.c_nstride8 == 8 && !p.R &&
                      p.relu_end == 0 &&
                      (p.ldc & 7) == 0 && (p.c_gstride & 7) == 0;
  if (big_ok && (int64_t)tiles(256, 128) * p.groups >= 256) tile = 256;
  else if ((int64_t)tiles(128, 128) * p.groups >= 192) tile = 128;  // 3/4 of the CUs busy beats 4x the tiles
  else if (p.full_n && p.N <= 128) tile = 96;                        // 64 x 128
  else tile = 64;
  return tile;
}

bool gemm_fuses_output(const GemmParams& p) {
  return p.M > 0 && p.N > 0 && p.nseg > 0 && choose_tile(p, p.seg[0].f32 != 0) == 256;
}

template <typename T, bool AF32>
static hipError_t launch_gemm_t(const GemmParams& p, hipStream_t st) {
  auto tiles = [&](int bm, int bn) { return ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn); };
  bool bk64 = p.K % 64 == 0;
  for (int s = 0; s < p.nseg; ++s) bk64 = bk64 && p.seg[s].k_end % 64 == 0;
  const int tile = choose_tile(p, AF32);
  if (p.ow && (tile != 256 || !p.opart || p.opart_ld < p.M)) return hipErrorInvalidValue;  // wide kernel only
  if (p.C2 && (tile == 256 || !p.out_f32 || p.groups != 1)) return hipErrorInvalidValue;  // small-tile kernel only
  const dim3 blk(256);
  if (tile == 256) {
    if constexpr (AF32) return hipErrorInvalidValue;  // excluded above
    else if (p.N % 256 == 0 && (int64_t)tiles(256, 256) * p.groups >= 256) {
      // 64-wide slices (half the block barriers) when every A segment allows them
      if (bk64)
        launch_k((gemm_big_kernel<T, 256, 256, 64, 2, 1>), dim3(big_grid(tiles(256, 256), 1), p.groups), dim3(512), 0,
                 st, p);
      else
        launch_k((gemm_big_kernel<T, 256, 256, 32, 3, 1>), dim3(big_grid(tiles(256, 256), 1), p.groups), dim3(512), 0,
                 st, p);
    }
    else launch_k((gemm_big_kernel<T, 256, 128, 32, 2, 2>), dim3(big_grid(tiles(256, 128), 2), p.groups), blk, 0, st, p);
  } else if (tile == 128) {
    if (bk64) launch_k((gemm_kernel<T, 128, 128, 2, 2, AF32, 64>), dim3(tiles(128, 128), p.groups), blk, 0, st, p);
    else launch_k((gemm_kernel<T, 128, 128, 2, 2, AF32, 32>), dim3(tiles(128, 128), p.groups), blk, 0, st, p);
  } else if (tile == 96) {
    if (bk64) launch_k((gemm_kernel<T, 64, 128, 2, 2, AF32, 64>), dim3(tiles(64, 128), p.groups), blk, 0, st, p);
    else launch_k((gemm_kernel<T, 64, 128, 2, 2, AF32, 32>), dim3(tiles(64, 128), p.groups), blk, 0, st, p);
  } else {
    if (bk64) launch_k((gemm_kernel<T, 64, 64, 2, 2, AF32, 64>), dim3(tiles(64, 64), p.groups), blk, 0, st, p);
    else launch_k((gemm_kernel<T, 64, 64, 2, 2, AF32, 32>), dim3(tiles(64, 64), p.groups), blk, 0, st, p);
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

// One thread per candidate: the partials of the fused last hidden layer summed in group order.
__global__ __launch_bounds__(256) void dlrm_logit_kernel(const float* __restrict__ part, int parts, int64_t ld, int M,
                                                         const float* __restrict__ b, float* __restrict__ logits,
                                                         float* __restrict__ out) {
  const int row = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (row >= M) return;
  float acc = 0.f;
  for (int c = 0; c < parts; ++c) acc += part[(int64_t)c * ld + row];
  const float z = acc + b[0];
  if (logits) logits[row] = z;
  out[row] = sigmoid_f32(z);
}

hipError_t launch_dlrm_logit(const float* part, int32_t parts, int64_t ld, int32_t M, const float* b, float* logits,
                             float* out, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (parts <= 0 || ld < M) return hipErrorInvalidValue;
  launch_k(dlrm_logit_kernel, dim3((M + 255) / 256), dim3(256), 0, st, part, parts, ld, M, b, logits, out);
  return hipGetLastError();
}

hipError_t launch_dlrm_output(const void* H, int32_t M, int32_t K, const void* w, const float* b,
                              float* logits, float* out, int lowp, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int blocks = (M + 3) / 4;
  if (lowp == 0)
    launch_k(dlrm_output_kernel<f16>, dim3(blocks), dim3(256), 0, st, (const f16*)H, M, K,
                       (const f16*)w, b, logits, out);
  else
    launch_k(dlrm_output_kernel<bf16>, dim3(blocks), dim3(256), 0, st, (const bf16*)H, M, K,
                       (const bf16*)w, b, logits, out);
  return hipGetLastError();
}

}  // namespace cvr
