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
// swiglu_kernel, per chunk of 32 positions (4 producer + 4 consumer waves):
//   1. gather: each position's 4 rows (fp32) -> clamp -> bf16 -> LDS tile E [32][128];
//   2. gate|up = W_gu E^T (MFMA 16x16x32, fp32 accumulate); producer w owns gate units
//      64w..64w+63 and the matching up units, so SiLU(gate+b) * (up+b) is formed in
//      registers and written to LDS as bf16 (the input of the down projection);
//   3. H = A W_down^T + b (MFMA 32x32x16; the bias starts one of the two accumulators),
//      rounded to bf16, staged through LDS and stored as rows; the rounded values are summed
//      per column over the chunk's positions for the mean pool (for a full chunk on the matrix
//      unit, as a product with a matrix of ones).
#include "chunk_plan.h"
#include "device_common.h"
#include "kernels.h"

namespace cvr {

// Exclusive scan of ceil(len / kSeqChunk) over the S*R segments (one block of 1024 threads):
// thread t owns a run of consecutive segments; the run totals are scanned within each wave by
// shuffles, then across the 16 waves.  Sums are 64-bit and every offset written is capped at
// max_chunks (what the workspace holds): with offsets that keep the layout contract the cap never
// binds; with offsets that break it (flagged by the expand kernel) the table stays monotone and
// every chunk it lists lies inside its own segment, so no later kernel leaves its arrays.
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* __restrict__ seq_offsets, int R, int S,
                                                           int64_t n_positions, int32_t max_chunks,
                                                           int32_t* __restrict__ chunk_off) {
  __shared__ long long wsum[16];
  const int SR = S * R;
  const int per = (SR + 1023) / 1024;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g0 = t * per;
  long long local = 0;
  for (int g = g0; g < g0 + per && g < SR; ++g) {
    int64_t a, e;
    segment_range(seq_offsets, R, g, n_positions, a, e);
    local += (e - a + kSeqChunk - 1) / kSeqChunk;
  }
  long long incl = local;  // inclusive scan within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    long long x = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const long long v = __shfl_up(x, off);
      if (lane >= off) x += v;
    }
    if (lane < 16) wsum[lane] = x;  // inclusive totals of waves 0..lane
  }
  __syncthreads();
  long long run = (w > 0 ? wsum[w - 1] : 0) + incl - local;  // exclusive prefix of this thread's run
  for (int g = g0; g < g0 + per && g < SR; ++g) {
    chunk_off[g] = (int32_t)(run < max_chunks ? run : max_chunks);
    int64_t a, e;
    segment_range(seq_offsets, R, g, n_positions, a, e);
    run += (e - a + kSeqChunk - 1) / kSeqChunk;
  }
  if (t == 1023) chunk_off[SR] = (int32_t)(wsum[15] < max_chunks ? wsum[15] : max_chunks);
}

// One descriptor per chunk: x = first position, y = (segment << 8) | positions in the chunk.
// One thread per chunk finds its segment by binary search over the chunk offsets.
__global__ __launch_bounds__(256) void chunk_desc_kernel(const int32_t* __restrict__ seq_offsets, int R, int S,
                                                         int64_t n_positions, const int32_t* __restrict__ chunk_off,
                                                         int2* __restrict__ desc) {
  const int SR = S * R;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunk_off[SR]) return;
  int lo = 0, hi = SR;  // chunk_off[lo] <= c < chunk_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_off[mid] <= c) lo = mid;
    else hi = mid;
  }
  int64_t a, e;
  segment_range(seq_offsets, R, lo, n_positions, a, e);
  const int64_t p0 = a + (int64_t)(c - chunk_off[lo]) * kSeqChunk;
  const int64_t left = e - p0;
  const int np = left > kSeqChunk ? kSeqChunk : (int)left;
  desc[c] = make_int2((int)p0, (lo << 8) | np);
}

int64_t chunk_plan_blocks(int64_t max_chunks) {
  const int64_t b = (max_chunks + 2047) / 2048;
  return b < 1 ? 1 : (b > 256 ? 256 : b);
}

hipError_t launch_chunk_table(const int32_t* seq_offsets, int R, int S, int64_t n_positions, int32_t* chunk_off,
                              int2* desc, hipStream_t st) {
  // every segment adds at most one partial chunk; the workspace holds this many
  const int64_t max_chunks = n_positions / kSeqChunk + (int64_t)S * R;
  if (max_chunks > INT32_MAX) return hipErrorInvalidValue;
  launch_k(chunk_table_kernel, dim3(1), dim3(1024), 0, st, seq_offsets, R, S, n_positions, (int32_t)max_chunks,
           chunk_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S * R == 0) return e;
  launch_k(chunk_desc_kernel, dim3((unsigned)((max_chunks + 255) / 256)), dim3(256), 0, st, seq_offsets, R, S,
           n_positions, chunk_off, desc);
  return hipGetLastError();
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Wait for every outstanding vector-memory operation of this wave (vmcnt(0); the other counters
// left alone).  Used right after the rare weight reloads, so that the compiler knows the weights
// have landed after the branch and puts no conservative full wait on the steady-state path,
// where it would also wait for the gathers and stores still in flight.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
typedef float float2_t __attribute__((ext_vector_type(2)));
constexpr int kD = 128;        // token width
constexpr int kHid = 256;      // SwiGLU hidden width
constexpr int kEPitch = kD + 8;
constexpr int kAPitch = kHid + 8;
constexpr int kM = kSeqChunk;  // positions per chunk = MFMA M tile
static_assert(kM == 32, "one 32-row MFMA tile per chunk");

// Persistent, producer/consumer: block b walks a contiguous range of n chunks with 8 waves.
// Waves 0-3 (producers) hold the gate|up weights of 64 hidden units each and turn E(c) into
// SiLU(gate) * up; they also write out the finished H rows and pool partials of chunk c-2.
// Waves 4-7 (consumers) hold the down projection for 32 output columns each, turn chunk c-1
// into bf16 H (staged in LDS) and pool partials, and gather and convert rows two chunks ahead.
// Every SIMD runs one wave of each kind, so one's VALU work overlaps the other's matrix
// instructions.  E, the SiLU tile and the H staging are double-buffered in LDS, the chunk
// descriptors sit in an eight-entry LDS ring; one block barrier per iteration hands them over.
// Loads and stores share one vector-memory counter and its waits are in issue order (a wait
// for one load also waits for every older one): consumers only load, in the same order on
// every path (ids of chunk c+4, then rows of chunk c+3), so the wait for the ids never covers
// the rows issued after them and the gathers keep two iterations to arrive; producers only
// store (they take no chunk data from global memory: descriptors come through LDS).
// Both roles pass the same n + 3 block barriers: one after the consumers' prologue and one at
// the end of each of the n + 2 pipeline iterations.
__global__ __launch_bounds__(512, 1) void swiglu_kernel(const SwigluParams p) {
  typedef bf16x8 V8;
  __shared__ __align__(16) bf16 Es[2][kM * kEPitch];
  __shared__ __align__(16) bf16 As[2][kM * kAPitch];
  __shared__ __align__(16) float Bs[4][2 * 64];          // producer w: gate bias, up bias
  __shared__ __align__(16) bf16 Hs[2][kM * kEPitch];     // finished H tile of a chunk
  __shared__ __align__(16) float Cs[2][kD];              // its pool partials
  // Descriptor ring: chunk c's descriptor sits in Dq[c % 8] from iteration c - 5 on (written
  // by one consumer thread a full iteration after it loaded it) until iteration c + 3.
  __shared__ int2 Dq[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool producer = wave < 4;
  const int rw = wave & 3;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  const int SR = p.S * p.R;
  // Offsets that break the layout contract (segments overlapping or out of order; flagged by the
  // expand kernel) can count more chunks than the workspace holds: never walk past that bound.
  const int total = p.chunk_off[SR] < p.max_chunks ? p.chunk_off[SR] : p.max_chunks;
  const int per = (total + gridDim.x - 1) / gridDim.x;
  const int c_begin = blockIdx.x * per;
  const int c_end = c_begin + per < total ? c_begin + per : total;
  const int n = c_end - c_begin;
  if (n <= 0) return;
  auto desc_of = [&](int i) { return p.desc[c_begin + (i < n ? i : n - 1)]; };

  if (producer) {
    // gate (h = 0) and up (h = 1) weights of unit group q (units 64w + 16q + lane%16), k step ks:
    // the 16x16x32 A operand, k = 32ks + 8(lane/16) .. +7
    V8 wg[4][2][kD / 32];
    float* bs = Bs[rw];
    int cur_s = -1;
    int2 dm1 = make_int2(0, 0), dm2 = make_int2(0, 0);  // descriptors of chunks i-1, i-2
    // chunk i-2 out: 32 rows x 128 columns of H (16 bytes per thread, twice) and partials
    // (nontemporal stores when the states outsize the last-level cache)
    auto store_out = [&](int i) {
      const int c = c_begin + i - 2;
      const int np = dm2.y & 255;
      const bf16* hsrc = Hs[i & 1];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int r = (tid >> 4) + 16 * q, ch = tid & 15;
        if (r < np) {
          const V8 v = *reinterpret_cast<const V8*>(&hsrc[r * kEPitch + ch * 8]);
          V8* dst = reinterpret_cast<V8*>(p.H + ((int64_t)dm2.x + r) * kD + ch * 8);
          if (p.nt) __builtin_nontemporal_store(v, dst);
          else *dst = v;
        }
      }
      if (tid < kD) {
        if (p.nt) __builtin_nontemporal_store(Cs[i & 1][tid], p.part + (int64_t)c * kD + tid);
        else p.part[(int64_t)c * kD + tid] = Cs[i & 1][tid];
      }
    };
    __syncthreads();  // E(0) and the first descriptors are in place
#pragma unroll 1
    for (int i = 0; i <= n + 1; ++i) {
      int2 d = make_int2(0, 0);
      if (i < n) {
        d = Dq[i & 7];
        const int s = (d.y >> 8) / p.R;
        if (s != cur_s) {
          const bf16* Wgu = p.Wgu + (int64_t)s * p.wgu_gstride;
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int u = h * kHid + rw * 64 + 16 * q + (lane & 15);
#pragma unroll
              for (int ks = 0; ks < kD / 32; ++ks)
                wg[q][h][ks] = *reinterpret_cast<const V8*>(Wgu + (int64_t)u * kD + 32 * ks + 8 * (lane >> 4));
            }
          const float* bgu = p.bgu + (int64_t)s * p.bgu_gstride + rw * 64 + lane;
          const float bg = bgu[0], bu = bgu[kHid];
          bs[lane] = bg;
          bs[64 + lane] = bu;
          cur_s = s;
          wait_vm_all();
        }
        const int b = i & 1;
        // Tiles of 16 hidden units x 16 positions (MFMA 16x16x32): unit group q, gate (h = 0) or
        // up (h = 1), positions 16pg .. +15.  Lane holds units 16q + 4(lane/16) + v, v = 0..3,
        // for position 16pg + lane%16; the accumulators start at the biases.
        f32x4 acc[4][2][2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4 bb = *reinterpret_cast<const float4*>(&bs[64 * h + 16 * q + 4 * (lane >> 4)]);
#pragma unroll
            for (int pg = 0; pg < 2; ++pg) acc[q][h][pg] = (f32x4){bb.x, bb.y, bb.z, bb.w};
          }
        V8 e[2][kD / 32];  // B operand: position 16pg + lane%16, k = 32ks + 8(lane/16) .. +7
#pragma unroll
        for (int pg = 0; pg < 2; ++pg)
#pragma unroll
          for (int ks = 0; ks < kD / 32; ++ks)
            e[pg][ks] = *reinterpret_cast<const V8*>(&Es[b][(16 * pg + (lane & 15)) * kEPitch + 32 * ks + 8 * (lane >> 4)]);
        // SiLU(gate) * up of element v of unit group q, positions 16pg + lane%16; four units of
        // one position leave as 8 bytes.  exp(-g) = exp2(-log2(e) * g).
        auto silu_v = [&](int q, int pg, int v) {
          const float g = acc[q][0][pg][v], u = acc[q][1][pg][v];
          const float e2 = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
          const float r = __builtin_amdgcn_rcpf(1.0f + e2);
          return (bf16)((g * u) * r);
        };
        auto silu_put = [&](int q, int pg) {
          bf16x4 o;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = silu_v(q, pg, v);
          *reinterpret_cast<bf16x4*>(&As[b][(16 * pg + (lane & 15)) * kAPitch + rw * 64 + 16 * q + 4 * (lane >> 4)]) = o;
        };
        auto mfma_step = [&](int q, int ks) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int pg = 0; pg < 2; ++pg)
              acc[q][h][pg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg[q][h][ks], e[pg][ks], acc[q][h][pg], 0, 0, 0);
        };
        // Unit group q's SiLU (vector and transcendental instructions) is interleaved with the
        // 16 matrix instructions of group q+1, one matrix instruction to four vector ones, so
        // that the vector work issues while the matrix unit is busy; only the last group's SiLU
        // runs on its own.
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks) mfma_step(0, ks);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 1; q < 4; ++q) {
#pragma unroll
          for (int ks = 0; ks < kD / 32; ++ks) mfma_step(q, ks);
          silu_put(q - 1, 0);
          silu_put(q - 1, 1);
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        silu_put(3, 0);
        silu_put(3, 1);
      }
      if (i >= 2) store_out(i);
      dm2 = dm1;
      dm1 = d;
      __syncthreads();
    }
    return;
  }

  // ---------------------------------------------------------------- consumers
  const int bt = tid - 256;  // 0..255
  // Global address space spelled out: a generic pointer would make these flat loads, which the
  // compiler cannot order against the row gathers and so waits for every load before them.
  typedef const __attribute__((address_space(1))) int32_t* gptr_i32;
  const gptr_i32 seq_ids = (gptr_i32)(p.seq_ids_ref ? *p.seq_ids_ref : p.seq_ids);
  // Granule i of a consumer thread covers position (bt + 256 i) / 32 and columns
  // 4 * (bt % 32) .. +3, which sit in one sequence column (table, rows and width fixed).
  const float* gtab;
  uint32_t grows, growb;  // rows of the column's table, bytes per row
  int gcol;
  {
    const int col = (bt & 31) * 4;
    int ci = 0;
#pragma unroll
    for (int cc = 1; cc < kMaxSeqCols; ++cc)
      if (cc < p.ncols && col >= p.col_off[cc]) ci = cc;
    gcol = ci;
    gtab = p.col_table[ci] + (col - p.col_off[ci]);
    grows = p.col_rows[ci] > 0x7fffffff ? 0x7fffffffu : (uint32_t)p.col_rows[ci];  // ids are int32
    growb = (uint32_t)p.col_dim[ci] * 4u;
  }
  const int gpos0 = bt >> 5;  // granule i is at position gpos0 + 8 i
  bool bad = false;
  auto load_ids = [&](int2 d, int32_t (&id)[4]) {
    const int np = d.y & 255;
    const gptr_i32 chunk_ids = seq_ids + (int64_t)d.x * p.ncols;  // the same for every lane
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = gpos0 + 8 * i;
      id[i] = chunk_ids[(pos < np ? pos : 0) * p.ncols + gcol];
    }
  };
  // Rows of positions past the chunk's length are loaded but never used: row m of H depends on
  // row m of E alone and such rows are neither stored nor summed.  An out-of-range id raises
  // the error flag and reads row 0 instead.  Such a position reads the id of the chunk's first
  // position, which is checked on its own account, so its check needs no length test.
  auto load_rows = [&](const int32_t (&id)[4], float4 (&row)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t r = (uint32_t)id[i];
      const bool ok = r < grows;
      bad |= !ok;
      row[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(gtab) + (uint64_t)(ok ? r : 0u) * growb);
    }
  };
  auto clampv = [&](float x) { return clamp_keep_nan(x, p.clamp); };
  auto convert = [&](const float4 (&row)[4], int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = bt + i * 256;
      bf16x4 o;
      o[0] = (bf16)clampv(row[i].x);
      o[1] = (bf16)clampv(row[i].y);
      o[2] = (bf16)clampv(row[i].z);
      o[3] = (bf16)clampv(row[i].w);
      *reinterpret_cast<bf16x4*>(&Es[b][(idx >> 5) * kEPitch + (idx & 31) * 4]) = o;
    }
  };

  V8 wd[kHid / 16];  // down projection: output column 32w + lane%32
  float bd = 0.f;
  int cur_s = -1;
  const int ncol = rw * 32 + lr;

  // Rows of chunks i+1 and i+2 and ids of i+3 in flight at the start of iteration i.
  // Descriptors come from the LDS ring: thread 0 loads chunk c's in iteration c - 6 and
  // publishes it at the start of iteration c - 5, before that iteration's loads, so the wait for
  // it never covers the gathers issued after it (vector-memory waits are in issue order).
  int32_t idsA[4], idsB[4];
  float4 rowA[4], rowB[4];
  int2 dload = make_int2(0, 0);  // thread 0: the descriptor of chunk i+5, loaded in iteration i-1
  {
    const int2 e0 = desc_of(0), e1 = desc_of(1), e2 = desc_of(2), e3 = desc_of(3);
    if (bt == 0) {
      Dq[0] = e0;
      Dq[1] = e1;
      Dq[2] = e2;
      Dq[3] = e3;
      Dq[4] = desc_of(4);
      dload = desc_of(5);
    }
    load_ids(e0, idsA);
    load_rows(idsA, rowA);
    load_ids(e1, idsA);
    convert(rowA, 0);
    load_rows(idsA, rowA);
    load_ids(e2, idsA);
    load_rows(idsA, rowB);
    load_ids(e3, idsA);
  }
  __syncthreads();  // E(0) and the ring complete (pairs with the producers' first wait)

  // Chunk c's H (the two accumulator chains h2) rounded to bf16 and staged in Hs[buf] for the
  // producers; its column sums over the chunk's positions go to Cs[buf].  Lane holds rows
  // 8*(v/4) + 4*(lane/32) + v%4 of column ncol, converted two rows at a time.
  auto epilogue = [&](const f32x16 (&h2)[2], int np, int buf) {
    bf16* hdst = Hs[buf];
    if (np == kM) {
      // The column sums of a full chunk on the matrix unit: a 32 x 16 matrix of ones times the
      // lane's rounded rows as the B operand (lanes l and l+32 hold the 32 rows of column l%32
      // between them, each row in one k slot), so every entry of the product is the sum.
      V8 hb[2];
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int m = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const bf16x2 h = __builtin_convertvector((float2_t){h2[0][v] + h2[1][v], h2[0][v + 1] + h2[1][v + 1]}, bf16x2);
        hdst[m * kEPitch + ncol] = h[0];
        hdst[(m + 1) * kEPitch + ncol] = h[1];
        hb[v >> 3][v & 7] = h[0];
        hb[v >> 3][(v & 7) + 1] = h[1];
      }
      V8 ones;
#pragma unroll
      for (int j = 0; j < 8; ++j) ones[j] = (bf16)1.0f;
      f32x16 cs = Lowp<bf16>::mfma32(ones, hb[0], (f32x16){});
      cs = Lowp<bf16>::mfma32(ones, hb[1], cs);
      if (lane < 32) Cs[buf][ncol] = cs[0];
    } else {
      // a partial chunk: only rows below np are summed, in row order per lane, then the two lanes
      float colsum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int m = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const bf16x2 h = __builtin_convertvector((float2_t){h2[0][v] + h2[1][v], h2[0][v + 1] + h2[1][v + 1]}, bf16x2);
        hdst[m * kEPitch + ncol] = h[0];
        hdst[(m + 1) * kEPitch + ncol] = h[1];
        if (m < np) colsum += (float)h[0];
        if (m + 1 < np) colsum += (float)h[1];
      }
      colsum += __shfl_xor(colsum, 32);
      if (lane < 32) Cs[buf][ncol] = colsum;
    }
  };

  // One pipeline iteration; `cur` holds the rows of chunk i+1 and is refilled with i+3 from the
  // ids in `use` (loaded the iteration before); `fill` receives the ids of chunk i+4.
  // Vector-memory waits are in issue order, so the loads go out as ids first, rows last: the
  // wait for this iteration's ids (next iteration, before its row loads) then does not cover
  // the rows issued after them, and rows keep two iterations to arrive.
  auto step = [&](int i, float4 (&cur)[4], int32_t (&use)[4], int32_t (&fill)[4]) {
    // E(i+1) and the gathers further ahead first: VALU work while the producer on this SIMD
    // runs its gate|up matrix instructions
    // The loads go out on every iteration (past the last chunk they repeat it, and what they
    // produce is not read), so that every path through the loop has the same vector-memory
    // operations in the same order and the compiler's waits count exactly how many are younger.
    if (bt == 0) {
      Dq[(i + 5) & 7] = dload;  // loaded an iteration ago; visible to all after this iteration's barrier
      dload = desc_of(i + 6);
    }
    const int2 d4 = Dq[(i + 4) & 7], dprev = Dq[(i - 1) & 7];
    load_ids(d4, fill);
    __builtin_amdgcn_sched_barrier(0);  // ids before rows
    convert(cur, (i + 1) & 1);
    load_rows(use, cur);
    if (i >= 1 && i <= n) {
      // chunk i-1: down projection on the SiLU tile, while the producer runs its SiLU
      const int s = (dprev.y >> 8) / p.R;
      if (s != cur_s) {
        const bf16* Wd = p.Wd + (int64_t)s * p.wd_gstride;
#pragma unroll
        for (int k = 0; k < kHid / 16; ++k) wd[k] = *reinterpret_cast<const V8*>(Wd + (int64_t)ncol * kHid + k * 16 + lk);
        bd = (p.bd + (int64_t)s * p.bd_gstride)[ncol];
        cur_s = s;
        wait_vm_all();
      }
      const bf16* A = As[(i - 1) & 1];
      f32x16 hacc[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {  // even and odd k in two accumulators, the even one starts at the bias
        hacc[0][v] = bd;
        hacc[1][v] = 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kHid / 16; ++k) {
        const V8 a = *reinterpret_cast<const V8*>(&A[lr * kAPitch + k * 16 + lk]);
        hacc[k & 1] = Lowp<bf16>::mfma32(a, wd[k], hacc[k & 1]);
      }
      // the first eight tile reads go out together, then one read after each matrix
      // instruction, so the chain does not wait on each read in turn
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      epilogue(hacc, dprev.y & 255, (i - 1) & 1);
    }
    __syncthreads();
  };
#pragma unroll 1
  for (int i = 0; i <= n + 1; i += 2) {
    step(i, rowA, idsA, idsB);
    if (i + 1 <= n + 1) step(i + 1, rowB, idsB, idsA);
  }
  if (bad) raise_flag(p.flag, ERRF_SEQ_ID_RANGE);
}

hipError_t launch_swiglu(const SwigluParams& p, int max_chunks, hipStream_t st) {
  if (max_chunks <= 0) return hipSuccess;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int blocks = max_chunks < cus ? max_chunks : cus;
  launch_k(swiglu_kernel, dim3(blocks), dim3(512), 0, st, p);
  return hipGetLastError();
}

// One wave per segment, four segments per block.  Lane l takes columns 4(l%32) .. +3 of chains
// 4(l/32) .. +3 (chunk c of the segment in chain c % 8, each chain summed in chunk order from
// zero), the four chains' next chunks in flight together; lane l then adds chains 0-3 in order
// and chains 4-7, fetched from lane l+32, after them: the order depends only on the segment's
// chunk count, so pools do not depend on the rest of the batch.
template <bool kNT>
__global__ __launch_bounds__(256) void seq_pool_kernel(const float* __restrict__ part, const int32_t* __restrict__ chunk_off,
                                                       const int32_t* __restrict__ seq_offsets, int R, int S,
                                                       int64_t n_positions, int32_t max_chunks,
                                                       float* __restrict__ pool, bf16* __restrict__ pool_bf) {
  const int lane = threadIdx.x & 63;
  // the last sequence's segments (the longest) first
  const int g = R * S - 1 - (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (g < 0) return;
  const int q = lane & 31, h = lane >> 5;
  const int s = g / R, r = g % R;
  int64_t a = seq_offsets[(int64_t)s * (R + 1) + r], e = seq_offsets[(int64_t)s * (R + 1) + r + 1];
  a = a < 0 ? 0 : (a > n_positions ? n_positions : a);
  e = e < a ? a : (e > n_positions ? n_positions : e);
  // chunk offsets past the workspace's chunk count come only from offsets the expand kernel flags
  const int c_lo = chunk_off[g] < max_chunks ? chunk_off[g] : max_chunks;
  const int c_hi = chunk_off[g + 1] < max_chunks ? chunk_off[g + 1] : max_chunks;
  float4 ch[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) ch[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  // four rounds of eight chunks at a time: sixteen loads in flight per lane
  for (int c = c_lo + 4 * h; c < c_hi; c += 32) {
    float4 v[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int cc = c + 8 * j + k;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (cc < c_hi) {
          const f32x4* src = reinterpret_cast<const f32x4*>(part + (int64_t)cc * kD + 4 * q);
          if constexpr (kNT) x = __builtin_nontemporal_load(src);
          else x = *src;
        }
        v[j][k] = make_float4(x[0], x[1], x[2], x[3]);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + 8 * j + k < c_hi) {
          ch[k].x += v[j][k].x;
          ch[k].y += v[j][k].y;
          ch[k].z += v[j][k].z;
          ch[k].w += v[j][k].w;
        }
  }
  // chains 4-7 from the upper half-wave
  float4 up[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    up[k].x = __shfl(ch[k].x, q + 32);
    up[k].y = __shfl(ch[k].y, q + 32);
    up[k].z = __shfl(ch[k].z, q + 32);
    up[k].w = __shfl(ch[k].w, q + 32);
  }
  if (h == 0) {
    float4 acc = ch[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      const float4 v = k < 4 ? ch[k] : up[k - 4];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const float len = (float)(e - a);
    const float4 o = e > a ? make_float4(acc.x / len, acc.y / len, acc.z / len, acc.w / len) : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(pool + (int64_t)g * kD + 4 * q) = o;
    if (pool_bf) {
      bf16x4 ob;
      ob[0] = (bf16)o.x;
      ob[1] = (bf16)o.y;
      ob[2] = (bf16)o.z;
      ob[3] = (bf16)o.w;
      *reinterpret_cast<bf16x4*>(pool_bf + (int64_t)g * kD + 4 * q) = ob;
    }
  }
}

hipError_t launch_seq_pool(const float* part, const int32_t* chunk_off, const int32_t* seq_offsets, int R, int S,
                           int64_t n_positions, int32_t max_chunks, float* pool, __bf16* pool_bf, bool nt,
                           hipStream_t st) {
  if (R * S <= 0) return hipSuccess;
  if (nt)
    launch_k(seq_pool_kernel<true>, dim3((R * S + 3) / 4), dim3(256), 0, st, part, chunk_off, seq_offsets, R, S,
             n_positions, max_chunks, pool, pool_bf);
  else
    launch_k(seq_pool_kernel<false>, dim3((R * S + 3) / 4), dim3(256), 0, st, part, chunk_off, seq_offsets, R, S,
             n_positions, max_chunks, pool, pool_bf);
  return hipGetLastError();
}

}  // namespace cvr
