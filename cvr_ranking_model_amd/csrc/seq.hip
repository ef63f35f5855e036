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
// swiglu_kernel, per chunk of 32 positions (8 waves):
//   1. gather: each position's 4 rows (fp32) -> clamp -> bf16 -> LDS tile E [32][128];
//   2. gate|up = W_gu E^T (MFMA 32x32x16, fp32 accumulate); wave w owns gate units
//      32w..32w+31 and the matching up units, so SiLU(gate+b) * (up+b) is formed in
//      registers and written to LDS as bf16 (the input of the down projection);
//   3. H = A W_down^T + b (MFMA 16x16x32), rounded to bf16, staged through LDS and stored as whole
//      rows; the rounded values are summed per column over the chunk's positions for the
//      mean pool.
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

// One descriptor per chunk: x = first position, y = (segment << 8) | positions in the chunk.
__global__ __launch_bounds__(256) void chunk_desc_kernel(const int32_t* __restrict__ seq_offsets, int R, int S,
                                                         int64_t n_positions, const int32_t* __restrict__ chunk_off,
                                                         int2* __restrict__ desc) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= S * R) return;
  const int s = g / R, r = g % R;
  int64_t a = seq_offsets[(int64_t)s * (R + 1) + r], e = seq_offsets[(int64_t)s * (R + 1) + r + 1];
  a = a < 0 ? 0 : (a > n_positions ? n_positions : a);
  e = e < a ? a : (e > n_positions ? n_positions : e);
  const int c0 = chunk_off[g], c1 = chunk_off[g + 1];
  for (int c = c0; c < c1; ++c) {
    const int64_t p0 = a + (int64_t)(c - c0) * kSeqChunk;
    const int64_t left = e - p0;
    const int np = left > kSeqChunk ? kSeqChunk : (int)left;
    desc[c] = make_int2((int)p0, (g << 8) | np);
  }
}

hipError_t launch_chunk_table(const int32_t* seq_offsets, int R, int S, int64_t n_positions, int32_t* chunk_off,
                              int2* desc, hipStream_t st) {
  launch_k(chunk_table_kernel, dim3(1), dim3(1024), 0, st, seq_offsets, R, S, n_positions, chunk_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S * R == 0) return e;
  launch_k(chunk_desc_kernel, dim3((S * R + 255) / 256), dim3(256), 0, st, seq_offsets, R, S, n_positions,
                     chunk_off, desc);
  return hipGetLastError();
}

constexpr int kD = 128;        // token width
constexpr int kHid = 256;      // SwiGLU hidden width
constexpr int kEPitch = kD + 8;
constexpr int kAPitch = kHid + 8;
constexpr int kM = kSeqChunk;  // positions per chunk = MFMA M tile
constexpr int kSwWaves = 8;    // two waves per SIMD
static_assert(kM == 32, "one 32-row MFMA tile per chunk");

// 16x16x32 bf16 MFMA: lane l holds A[l%16][8(l/16)..+7] and B[8(l/16)..+7][l%16] and gets
// D[4(l/16)+v][l%16], v = 0..3.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Persistent: block b walks a contiguous range of chunks with 8 waves (two per SIMD, so one
// wave's VALU work and waits overlap the other's matrix instructions).  Each wave keeps its
// share of the sequence's weights in registers and reloads them only when the range crosses
// into another sequence: 32 gate + 32 up hidden units (gate|up as 2 MFMA 32x32x16 tiles x 8
// k-steps) and 16 output columns of the down projection (MFMA 16x16x32 over 2 position tiles
// x 8 k-steps).
// Order of one iteration (chunk c): MFMAs on E(c) -> H(c) in registers; convert the rows of
// c+1 (requested one iteration earlier) into the other E buffer; request the rows of c+2, the
// ids of c+3 and the descriptor of c+4; stage H(c) through LDS and store it.  Loads and
// stores share one vector-memory counter, so every wait for loads comes a whole iteration
// after the last stores.
__global__ __launch_bounds__(kSwWaves * 64, 1) void swiglu_kernel(const SwigluParams p) {
  typedef bf16x8 V8;
  constexpr int NT = kSwWaves * 64;
  constexpr int NG = kM * kD / 4 / NT;  // float4 granules per thread per chunk
  __shared__ __align__(16) bf16 Es[2][kM * kEPitch];
  __shared__ __align__(16) bf16 As[kM * kAPitch];   // SiLU(gate) * up, then the staged H tile
  __shared__ __align__(16) float Bgu[2 * kHid];     // gate then up biases of the current sequence

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  const int l16 = lane & 15, lq = lane >> 4;
  const int SR = p.S * p.R;
  const int total = p.chunk_off[SR];
  const int per = (total + gridDim.x - 1) / gridDim.x;
  const int c_begin = blockIdx.x * per;
  const int c_end = c_begin + per < total ? c_begin + per : total;
  if (c_begin >= c_end) return;

  // Granule i of a thread covers position (tid + NT i) / 32 and columns 4 * (tid % 32) .. +3,
  // which sit in one sequence column; its table, row count and row width are fixed.
  const float* gtab;
  int64_t grows;
  int gstride, gcol;
  {
    const int col = (tid & 31) * 4;
    int ci = 0;
#pragma unroll
    for (int cc = 1; cc < kMaxSeqCols; ++cc)
      if (cc < p.ncols && col >= p.col_off[cc]) ci = cc;
    gcol = ci;
    gtab = p.col_table[ci] + (col - p.col_off[ci]);
    grows = p.col_rows[ci];
    gstride = p.col_dim[ci];
  }
  const int gpos0 = tid >> 5;  // position of granule 0; granule i is at gpos0 + (NT/32) i
  bool bad = false;
  auto desc_of = [&](int c) { return p.desc[c < c_end ? c : c_end - 1]; };
  auto load_ids = [&](int2 d, int32_t (&id)[NG]) {
    const int np = d.y & 255;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int pos = gpos0 + (NT / 32) * i;
      id[i] = p.seq_ids[((int64_t)d.x + (pos < np ? pos : 0)) * p.ncols + gcol];
    }
  };
  auto load_rows = [&](int2 d, const int32_t (&id)[NG], float4 (&row)[NG]) {
    const int np = d.y & 255;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int32_t r = id[i];
      const bool live = gpos0 + (NT / 32) * i < np;
      const bool ok = r >= 0 && (int64_t)r < grows;
      if (!ok && live) bad = true;
      row[i] = *reinterpret_cast<const float4*>(gtab + (int64_t)(ok ? r : 0) * gstride);
      if (!ok || !live) row[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  // clamp + bf16 of a chunk's rows into E buffer b
  auto convert = [&](const float4 (&row)[NG], int b) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int idx = tid + i * NT;
      bf16x4 o;
      o[0] = (bf16)clamp_keep_nan(row[i].x, p.clamp);
      o[1] = (bf16)clamp_keep_nan(row[i].y, p.clamp);
      o[2] = (bf16)clamp_keep_nan(row[i].z, p.clamp);
      o[3] = (bf16)clamp_keep_nan(row[i].w, p.clamp);
      *reinterpret_cast<bf16x4*>(&Es[b][(idx >> 5) * kEPitch + (idx & 31) * 4]) = o;
    }
  };

  V8 wg[2][kD / 16];   // gate tile (units 32w..32w+31) and the matching up tile
  V8 wd[kHid / 32];    // down projection: output column 16w + lane%16, k = 32 ks + 8 (lane/16)
  float bd = 0.f;
  int cur_s = -1;
  auto load_weights = [&](int s) {
    const bf16* Wgu = p.Wgu + (int64_t)s * p.wgu_gstride;
    const float* bgu = p.bgu + (int64_t)s * p.bgu_gstride;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = j * kHid + wave * 32 + lr;
#pragma unroll
      for (int k = 0; k < kD / 16; ++k) wg[j][k] = *reinterpret_cast<const V8*>(Wgu + (int64_t)n * kD + k * 16 + lk);
    }
    __syncthreads();  // no wave still reads the previous sequence's biases
    for (int h = tid; h < 2 * kHid; h += NT) Bgu[h] = bgu[h];
    const bf16* Wd = p.Wd + (int64_t)s * p.wd_gstride;
    const int n = wave * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < kHid / 32; ++ks) wd[ks] = *reinterpret_cast<const V8*>(Wd + (int64_t)n * kHid + ks * 32 + lq * 8);
    bd = (p.bd + (int64_t)s * p.bd_gstride)[n];
    cur_s = s;
  };

  // Prologue: E(c_begin) in buffer 0, rows of c_begin+1 and ids of c_begin+2 in flight.
  int2 dc = desc_of(c_begin), d1 = desc_of(c_begin + 1), d2 = desc_of(c_begin + 2), d3 = desc_of(c_begin + 3);
  int32_t ids[NG];
  float4 row[NG];
  load_ids(dc, ids);
  load_rows(dc, ids, row);
  load_ids(d1, ids);
  convert(row, 0);
  load_rows(d1, ids, row);
  load_ids(d2, ids);
  int buf = 0;
#pragma unroll 1
  for (int c = c_begin; c < c_end; ++c) {
    const int seg = dc.y >> 8, np = dc.y & 255;
    const int64_t p0 = dc.x;
    const int s = seg / p.R;
    if (s != cur_s) load_weights(s);
    __syncthreads();  // E(c) complete; As free

    // gate|up for this wave's 32 hidden units, computed transposed (hidden units x
    // positions) so each lane ends with four consecutive hidden units of one position:
    // SiLU(gate) * up for them leaves as one 8-byte LDS write.
    {
      f32x16 acc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
#pragma unroll
      for (int k = 0; k < kD / 16; ++k) {
        const V8 e = *reinterpret_cast<const V8*>(&Es[buf][lr * kEPitch + k * 16 + lk]);
        acc[0] = Lowp<bf16>::mfma32(wg[0][k], e, acc[0]);
        acc[1] = Lowp<bf16>::mfma32(wg[1][k], e, acc[1]);
      }
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        // rows 8*v4 + 4*(lane/32) .. +3 of the tile are hidden units; column lr is the position
        const int h0 = wave * 32 + 8 * v4 + 4 * (lane >> 5);
        const float4 bg4 = *reinterpret_cast<const float4*>(&Bgu[h0]);
        const float4 bu4 = *reinterpret_cast<const float4*>(&Bgu[kHid + h0]);
        const float bgv[4] = {bg4.x, bg4.y, bg4.z, bg4.w};
        const float buv[4] = {bu4.x, bu4.y, bu4.z, bu4.w};
        bf16x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = acc[0][4 * v4 + q] + bgv[q];
          const float u = acc[1][4 * v4 + q] + buv[q];
          const float sg = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
          o[q] = (bf16)(sg * u);
        }
        *reinterpret_cast<bf16x4*>(&As[lr * kAPitch + h0]) = o;
      }
    }
    __syncthreads();

    // down projection for output columns 16w .. 16w+15: two 16-position tiles
    f32x4 acc2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc2[t][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kHid / 32; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const V8 a = *reinterpret_cast<const V8*>(&As[(16 * t + l16) * kAPitch + ks * 32 + lq * 8]);
        acc2[t] = mfma16(a, wd[ks], acc2[t]);
      }
    }

    // next chunk's E; then the gathers two and three chunks ahead go out before any store
    convert(row, buf ^ 1);
    load_rows(d2, ids, row);
    load_ids(d3, ids);
    const int2 d4 = desc_of(c + 4);  // used next iteration, so its load latency stays hidden

    // H(c): round to bf16, column sums for the mean pool, stage rows in As, 16-byte stores.
    // Lane holds rows 16t + 4(lane/16) + v of column 16w + lane%16.
    __syncthreads();  // every wave is done reading As
    const int n = wave * 16 + l16;
    float colsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * t + 4 * lq + v;
        const bf16 h = (bf16)(acc2[t][v] + bd);
        As[m * kAPitch + n] = h;
        if (m < np) colsum += (float)h;
      }
    colsum += __shfl_xor(colsum, 16);
    colsum += __shfl_xor(colsum, 32);
    if (lane < 16) p.part[(int64_t)c * kD + n] = colsum;
    __syncthreads();
    {
      const int r = tid >> 4, ch = tid & 15;
      if (r < np)
        *reinterpret_cast<V8*>(p.H + (p0 + r) * kD + ch * 8) = *reinterpret_cast<const V8*>(&As[r * kAPitch + ch * 8]);
    }
    dc = d1;
    d1 = d2;
    d2 = d3;
    d3 = d4;
    buf ^= 1;
  }
  if (bad) raise_flag(p.flag, ERRF_SEQ_ID_RANGE);
}

hipError_t launch_swiglu(const SwigluParams& p, int max_chunks, hipStream_t st) {
  if (max_chunks <= 0) return hipSuccess;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int blocks = max_chunks < cus ? max_chunks : cus;
  launch_k(swiglu_kernel, dim3(blocks), dim3(kSwWaves * 64), 0, st, p);
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
  launch_k(seq_pool_kernel, dim3(R * S), dim3(kD), 0, st, part, chunk_off, seq_offsets, R, S, n_positions, pool);
  return hipGetLastError();
}

}  // namespace cvr
