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
// swiglu_kernel, per chunk of 32 positions (4 waves):
//   1. gather: each position's 4 rows (fp32) -> clamp -> bf16 -> LDS tile E [32][128];
//   2. gate|up = W_gu E^T (MFMA 32x32x16, fp32 accumulate); wave w owns gate units
//      64w..64w+63 and the matching up units, so SiLU(gate+b) * (up+b) is formed in
//      registers and written to LDS as bf16 (the input of the down projection);
//   3. H = A W_down^T + b (MFMA), rounded to bf16, staged through LDS and stored as whole
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
static_assert(kM == 32, "one 32-row MFMA tile per chunk");

// Persistent: block b walks a contiguous range of chunks; each wave keeps its share of the
// sequence's weights in registers (gate/up: 2+2 unit tiles x 8 k-steps; down: 1 column tile x
// 16 k-steps) and reloads them only when the range crosses into another sequence.
// Order of one iteration (chunk c): MFMAs on E(c) -> H(c) in registers; convert the rows of
// c+1 (requested one iteration earlier) into the other E buffer; request the rows of c+2, the
// ids of c+3 and the descriptor of c+4; stage H(c) through LDS and store it.  Loads and stores share one vector-
// memory counter, so every wait for loads comes a whole iteration after the last stores.
__global__ __launch_bounds__(256, 1) void swiglu_kernel(const SwigluParams p) {
  typedef bf16x8 V8;
  __shared__ __align__(16) bf16 Es[2][kM * kEPitch];
  __shared__ __align__(16) bf16 As[kM * kAPitch];   // SiLU(gate) * up, then the staged H tile
  __shared__ __align__(16) float Bgu[2 * kHid];     // gate then up biases of the current sequence

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  const int SR = p.S * p.R;
  const int total = p.chunk_off[SR];
  const int per = (total + gridDim.x - 1) / gridDim.x;
  const int c_begin = blockIdx.x * per;
  const int c_end = c_begin + per < total ? c_begin + per : total;
  if (c_begin >= c_end) return;

  // Each thread owns 4 float4 granules of the 32x128 chunk tile: granule i covers position
  // (tid + 256 i) / 32 and columns 4 * ((tid + 256 i) % 32) .. +3, which sit in one sequence
  // column; its table, row count and row width are fixed for the kernel.
  const float* gtab[4];
  int64_t grows[4];
  int gstride[4], gcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int col = ((tid + i * 256) & 31) * 4;
    int ci = 0;
#pragma unroll
    for (int cc = 1; cc < kMaxSeqCols; ++cc)
      if (cc < p.ncols && col >= p.col_off[cc]) ci = cc;
    gcol[i] = ci;
    gtab[i] = p.col_table[ci] + (col - p.col_off[ci]);
    grows[i] = p.col_rows[ci];
    gstride[i] = p.col_dim[ci];
  }
  const int gpos0 = tid >> 5;  // position of granule 0; granule i is at gpos0 + 8 i
  bool bad = false;
  auto desc_of = [&](int c) { return p.desc[c < c_end ? c : c_end - 1]; };
  auto load_ids = [&](int2 d, int32_t (&id)[4]) {
    const int np = d.y & 255;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = gpos0 + 8 * i;
      id[i] = p.seq_ids[((int64_t)d.x + (pos < np ? pos : 0)) * p.ncols + gcol[i]];
    }
  };
  auto load_rows = [&](int2 d, const int32_t (&id)[4], float4 (&row)[4]) {
    const int np = d.y & 255;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t r = id[i];
      const bool live = gpos0 + 8 * i < np;
      const bool ok = r >= 0 && (int64_t)r < grows[i];
      if (!ok && live) bad = true;
      row[i] = *reinterpret_cast<const float4*>(gtab[i] + (int64_t)(ok ? r : 0) * gstride[i]);
      if (!ok || !live) row[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  // clamp + bf16 of a chunk's rows into E buffer b
  auto convert = [&](const float4 (&row)[4], int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + i * 256;
      bf16x4 o;
      o[0] = (bf16)clamp_keep_nan(row[i].x, p.clamp);
      o[1] = (bf16)clamp_keep_nan(row[i].y, p.clamp);
      o[2] = (bf16)clamp_keep_nan(row[i].z, p.clamp);
      o[3] = (bf16)clamp_keep_nan(row[i].w, p.clamp);
      *reinterpret_cast<bf16x4*>(&Es[b][(idx >> 5) * kEPitch + (idx & 31) * 4]) = o;
    }
  };

  V8 wg[4][kD / 16];   // gate tiles 0,1 and up tiles 2,3 of this wave
  V8 wd[kHid / 16];    // down projection, output columns 32*wave..32*wave+31
  float bd = 0.f;
  int cur_s = -1;
  auto load_weights = [&](int s) {
    const bf16* Wgu = p.Wgu + (int64_t)s * p.wgu_gstride;
    const float* bgu = p.bgu + (int64_t)s * p.bgu_gstride;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = (j < 2 ? 0 : kHid) + wave * 64 + (j & 1) * 32 + lr;
#pragma unroll
      for (int k = 0; k < kD / 16; ++k) wg[j][k] = *reinterpret_cast<const V8*>(Wgu + (int64_t)n * kD + k * 16 + lk);
    }
    __syncthreads();  // no wave still reads the previous sequence's biases
    for (int h = tid; h < 2 * kHid; h += 256) Bgu[h] = bgu[h];
    const bf16* Wd = p.Wd + (int64_t)s * p.wd_gstride;
    const int n = wave * 32 + lr;
#pragma unroll
    for (int k = 0; k < kHid / 16; ++k) wd[k] = *reinterpret_cast<const V8*>(Wd + (int64_t)n * kHid + k * 16 + lk);
    bd = (p.bd + (int64_t)s * p.bd_gstride)[n];
    cur_s = s;
  };

  // Prologue: E(c_begin) in buffer 0, rows of c_begin+1 and ids of c_begin+2 in flight.
  int2 dc = desc_of(c_begin), d1 = desc_of(c_begin + 1), d2 = desc_of(c_begin + 2), d3 = desc_of(c_begin + 3);
  int32_t ids[4];
  float4 row[4];
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

    // gate|up for this wave's 64 hidden units, computed transposed (hidden units x
    // positions) so each lane ends with four consecutive hidden units of one position:
    // SiLU(gate) * up for them leaves as one 8-byte LDS write.
    {
      f32x16 acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
#pragma unroll
      for (int k = 0; k < kD / 16; ++k) {
        const V8 e = *reinterpret_cast<const V8*>(&Es[buf][lr * kEPitch + k * 16 + lk]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = Lowp<bf16>::mfma32(wg[j][k], e, acc[j]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          // rows 8*v4 + 4*(lane/32) .. +3 of tile j are hidden units; column lr is the position
          const int h0 = wave * 64 + j * 32 + 8 * v4 + 4 * (lane >> 5);
          const float4 bg4 = *reinterpret_cast<const float4*>(&Bgu[h0]);
          const float4 bu4 = *reinterpret_cast<const float4*>(&Bgu[kHid + h0]);
          const float bgv[4] = {bg4.x, bg4.y, bg4.z, bg4.w};
          const float buv[4] = {bu4.x, bu4.y, bu4.z, bu4.w};
          bf16x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = acc[j][4 * v4 + q] + bgv[q];
            const float u = acc[j + 2][4 * v4 + q] + buv[q];
            const float sg = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
            o[q] = (bf16)(sg * u);
          }
          *reinterpret_cast<bf16x4*>(&As[lr * kAPitch + h0]) = o;
        }
    }
    __syncthreads();

    // down projection -> H (fp32 accumulators); even and odd k steps accumulate separately
    // so consecutive MFMAs do not wait on each other
    f32x16 acc2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc2[h][v] = 0.f;
#pragma unroll
    for (int k = 0; k < kHid / 16; ++k) {
      const V8 a = *reinterpret_cast<const V8*>(&As[lr * kAPitch + k * 16 + lk]);
      acc2[k & 1] = Lowp<bf16>::mfma32(a, wd[k], acc2[k & 1]);
    }

    // next chunk's E; then the gathers two and three chunks ahead go out before any store
    convert(row, buf ^ 1);
    load_rows(d2, ids, row);
    load_ids(d3, ids);
    const int2 d4 = desc_of(c + 4);  // used next iteration, so its load latency stays hidden

    // H(c): round to bf16, column sums for the mean pool, stage rows in As, 16-byte stores
    __syncthreads();  // every wave is done reading As
    const int n = wave * 32 + lr;
    float colsum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const bf16 h = (bf16)((acc2[0][v] + acc2[1][v]) + bd);
      As[m * kAPitch + n] = h;
      if (m < np) colsum += (float)h;
    }
    colsum += __shfl_xor(colsum, 32);
    if (lane < 32) p.part[(int64_t)c * kD + n] = colsum;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (tid >> 4) + 16 * i, ch = tid & 15;
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
  launch_k(swiglu_kernel, dim3(blocks), dim3(256), 0, st, p);
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
