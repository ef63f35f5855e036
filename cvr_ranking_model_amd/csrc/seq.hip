// Behaviour-sequence encoding of the CVR model (steps B3-B5).
//
// The CVR article (sections 3.2.1-3.2.3) represents each behaviour as the concat of its
// item-ID, action-type, timestamp and side-info embeddings, fetched from tables the three
// sequences share, and maps every position of each sequence into the common latent space
// with that sequence's own SwiGLU network (linear in the sequence length).
//
// Work is cut into chunks of up to kSeqChunk positions that never cross from one
// (sequence, request) segment into the next, so the per-chunk column sums of the encoded
// states reduce to each segment's mean pool in a fixed order (bitwise reproducible).
//
// swiglu_kernel, per chunk (4 waves):
//   1. gather: each position's 4 rows (fp32) -> clamp -> bf16 -> LDS tile E [64][128];
//   2. gate|up = E W_gu^T (MFMA 32x32x16, fp32 accumulate); wave w owns gate columns
//      64w..64w+63 and the matching up columns, so SiLU(gate+b) * (up+b) is formed in
//      registers and written to LDS as bf16 (the input of the down projection);
//   3. H = A W_down^T + b (MFMA), rounded to bf16 and stored; the rounded values are
//      summed per column over the chunk's positions for the mean pool.
#include "device_common.h"
#include "kernels.h"

namespace cvr {

// Exclusive scan of ceil(len / kSeqChunk) over the S*R segments (one block).
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* __restrict__ seq_offsets, int R, int S,
                                                           int64_t n_positions, int32_t* __restrict__ chunk_off) {
  __shared__ int32_t part[1024];
  const int SR = S * R;
  const int per = (SR + 1023) / 1024;
  const int t = threadIdx.x;
  const int g0 = t * per;
  int32_t local = 0;
  for (int g = g0; g < g0 + per && g < SR; ++g) {
    const int s = g / R, r = g % R;
    int64_t a = seq_offsets[(int64_t)s * (R + 1) + r], b = seq_offsets[(int64_t)s * (R + 1) + r + 1];
    a = a < 0 ? 0 : (a > n_positions ? n_positions : a);
    b = b < a ? a : (b > n_positions ? n_positions : b);
    local += (int32_t)((b - a + kSeqChunk - 1) / kSeqChunk);
  }
  part[t] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t run = part[t] - local;  // exclusive prefix of this thread's range
  for (int g = g0; g < g0 + per && g < SR; ++g) {
    chunk_off[g] = run;
    const int s = g / R, r = g % R;
    int64_t a = seq_offsets[(int64_t)s * (R + 1) + r], b = seq_offsets[(int64_t)s * (R + 1) + r + 1];
    a = a < 0 ? 0 : (a > n_positions ? n_positions : a);
    b = b < a ? a : (b > n_positions ? n_positions : b);
    run += (int32_t)((b - a + kSeqChunk - 1) / kSeqChunk);
  }
  if (t == 1023) chunk_off[SR] = part[1023];
}

hipError_t launch_chunk_table(const int32_t* seq_offsets, int R, int S, int64_t n_positions, int32_t* chunk_off,
                              hipStream_t st) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, st, seq_offsets, R, S, n_positions, chunk_off);
  return hipGetLastError();
}

// Segment (s*R + r) and position range of chunk b, or false if b is past the last chunk.
__device__ __forceinline__ bool locate_chunk(const int32_t* __restrict__ chunk_off, const int32_t* __restrict__ seq_offsets,
                                             int R, int S, int64_t n_positions, int b, int& seg, int64_t& p0, int& np) {
  const int SR = S * R;
  if (b >= chunk_off[SR]) return false;
  int lo = 0, hi = SR - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_off[mid] <= b) lo = mid; else hi = mid - 1;
  }
  seg = lo;
  const int s = lo / R, r = lo % R;
  int64_t a = seq_offsets[(int64_t)s * (R + 1) + r], e = seq_offsets[(int64_t)s * (R + 1) + r + 1];
  a = a < 0 ? 0 : (a > n_positions ? n_positions : a);
  e = e < a ? a : (e > n_positions ? n_positions : e);
  p0 = a + (int64_t)(b - chunk_off[lo]) * kSeqChunk;
  const int64_t left = e - p0;
  np = left > kSeqChunk ? kSeqChunk : (int)left;
  return np > 0;
}

constexpr int kD = 128;        // token width
constexpr int kHid = 256;      // SwiGLU hidden width
constexpr int kEPitch = kD + 8;
constexpr int kAPitch = kHid + 8;

__global__ __launch_bounds__(256) void swiglu_kernel(const SwigluParams p) {
  typedef bf16x8 V8;
  __shared__ __align__(16) bf16 Es[kSeqChunk * kEPitch];
  __shared__ __align__(16) bf16 As[kSeqChunk * kAPitch];

  int seg, np;
  int64_t p0;
  if (!locate_chunk(p.chunk_off, p.seq_offsets, p.R, p.S, p.n_positions, blockIdx.x, seg, p0, np)) return;
  const int s = seg / p.R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // 1. gather + clamp + bf16 into Es (float4 granules: 64 positions x 32 granules)
  bool bad = false;
#pragma unroll
  for (int i = 0; i < (kSeqChunk * kD / 4) / 256; ++i) {
    const int idx = tid + i * 256;
    const int pos = idx >> 5;
    const int col = (idx & 31) * 4;
    int ci = 0;
#pragma unroll
    for (int c = 1; c < kMaxSeqCols; ++c)
      if (c < p.ncols && col >= p.col_off[c]) ci = c;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (pos < np) {
      const int32_t id = p.seq_ids[(p0 + pos) * p.ncols + ci];
      if (id >= 0 && (int64_t)id < p.col_rows[ci])
        v = *reinterpret_cast<const float4*>(p.col_table[ci] + (int64_t)id * p.col_dim[ci] + (col - p.col_off[ci]));
      else
        bad = true;
    }
    bf16x4 o;
    o[0] = (bf16)clamp_keep_nan(v.x, p.clamp);
    o[1] = (bf16)clamp_keep_nan(v.y, p.clamp);
    o[2] = (bf16)clamp_keep_nan(v.z, p.clamp);
    o[3] = (bf16)clamp_keep_nan(v.w, p.clamp);
    *reinterpret_cast<bf16x4*>(&Es[pos * kEPitch + col]) = o;
  }
  if (bad) raise_flag(p.flag, ERRF_SEQ_ID_RANGE);
  __syncthreads();

  const int lr = lane & 31, lk = (lane >> 5) * 8;
  const bf16* Wgu = p.Wgu + (int64_t)s * p.wgu_gstride;   // [512][128]: gate rows 0..255, up rows 256..511
  const float* bgu = p.bgu + (int64_t)s * p.bgu_gstride;  // [512]
  // 2. gate|up for this wave's 64 hidden units
  {
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
#pragma unroll
    for (int k = 0; k < kD; k += 16) {
      V8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const V8*>(&Es[(i * 32 + lr) * kEPitch + k + lk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = (j < 2 ? 0 : kHid) + wave * 64 + (j & 1) * 32 + lr;
        b[j] = *reinterpret_cast<const V8*>(Wgu + (int64_t)n * kD + k + lk);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = Lowp<bf16>::mfma32(a[i], b[j], acc[i][j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wave * 64 + j * 32 + lr;  // hidden unit
      const float bg = bgu[n], bu = bgu[kHid + n];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const float g = acc[i][j][v] + bg;
          const float u = acc[i][j + 2][v] + bu;
          const float sg = g / (1.0f + expf(-g));
          As[m * kAPitch + n] = (bf16)(sg * u);
        }
    }
  }
  __syncthreads();

  // 3. down projection: wave w owns output columns 32w..32w+31
  const bf16* Wd = p.Wd + (int64_t)s * p.wd_gstride;  // [128][256]
  const float* bd = p.bd + (int64_t)s * p.bd_gstride;
  f32x16 acc2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc2[i][v] = 0.f;
  const int n = wave * 32 + lr;
#pragma unroll 4
  for (int k = 0; k < kHid; k += 16) {
    const V8 b = *reinterpret_cast<const V8*>(Wd + (int64_t)n * kHid + k + lk);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const V8 a = *reinterpret_cast<const V8*>(&As[(i * 32 + lr) * kAPitch + k + lk]);
      acc2[i] = Lowp<bf16>::mfma32(a, b, acc2[i]);
    }
  }
  const float bn = bd[n];
  float colsum = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (m < np) {
        const bf16 h = (bf16)(acc2[i][v] + bn);
        p.H[(p0 + m) * kD + n] = h;
        colsum += (float)h;
      }
    }
  colsum += __shfl_xor(colsum, 32);
  if (lane < 32) p.part[(int64_t)blockIdx.x * kD + n] = colsum;
}

hipError_t launch_swiglu(const SwigluParams& p, int max_chunks, hipStream_t st) {
  if (max_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_kernel, dim3(max_chunks), dim3(256), 0, st, p);
  return hipGetLastError();
}

// Mean pool per segment: sum the chunk partials in chunk order, divide by the length.
__global__ __launch_bounds__(128) void seq_pool_kernel(const float* __restrict__ part, const int32_t* __restrict__ chunk_off,
                                                       const int32_t* __restrict__ seq_offsets, int R, int S,
                                                       int64_t n_positions, float* __restrict__ pool) {
  const int g = blockIdx.x;
  const int j = threadIdx.x;
  const int s = g / R, r = g % R;
  int64_t a = seq_offsets[(int64_t)s * (R + 1) + r], e = seq_offsets[(int64_t)s * (R + 1) + r + 1];
  a = a < 0 ? 0 : (a > n_positions ? n_positions : a);
  e = e < a ? a : (e > n_positions ? n_positions : e);
  float acc = 0.f;
  for (int c = chunk_off[g]; c < chunk_off[g + 1]; ++c) acc += part[(int64_t)c * kD + j];
  const float v = e > a ? acc / (float)(e - a) : 0.f;
  pool[(int64_t)g * kD + j] = v;
}

hipError_t launch_seq_pool(const float* part, const int32_t* chunk_off, const int32_t* seq_offsets, int R, int S,
                           int64_t n_positions, float* pool, hipStream_t st) {
  if (R * S <= 0) return hipSuccess;
  hipLaunchKernelGGL(seq_pool_kernel, dim3(R * S), dim3(kD), 0, st, part, chunk_off, seq_offsets, R, S, n_positions, pool);
  return hipGetLastError();
}

}  // namespace cvr
