// Query Boosting token mixer, fused (step B8; CVR article section 3.2.3).
//
// The N + 3 tokens of a candidate (16 x 128, fp32) are split into 16 heads of 8 columns;
// mixed token h concatenates head h of every token (16 x 8 = 128 values), goes through its
// own FFN 128 -> 256 (ReLU) -> 128, and the result is scattered back (revert) onto head h of
// every token and added to the input: Z[t][8h + j] = Y[t][8h + j] + F_h[8t + j].
//
// One block of 8 waves per (head h, run of 64-candidate tiles), one block per CU.  Waves 0-3
// hold the first Linear's weights and waves 4-7 the second's, each in MFMA operand registers,
// loaded once for the whole run.  The tiles of the run go through a two-stage pipeline: at
// stage s waves 0-3 compute tile s's hidden activations while waves 4-7 finish tile s - 1, and
// every wave has tile s + 1's tokens in flight.  Token and hidden tiles are double-buffered in
// LDS; a stage ends with two block barriers (results handed over, then the next tokens stored).
//   1. split + mix: Y[c][t][8h .. 8h+7] of the tile's 64 candidates sit in LDS as fp32;
//   2. the first Linear as a transposed product, hidden^T = W1 X^T (MFMA 32x32x16, fp32
//      accumulation), X rounded to bf16 (the Linear input rounding) as its fragments are read:
//      each lane ends with 4 consecutive hidden units of one candidate, adds the bias, applies
//      ReLU, rounds to bf16 and stores them to LDS as 8 bytes;
//   3. the second Linear the same way, F^T = W2 hidden^T: each lane ends with 4 consecutive
//      outputs 8t + j .. 8t + j + 3, which revert to 4 consecutive columns of token t; the
//      epilogue adds the bias, then the residual (from the fp32 tile in LDS), and writes 16
//      bytes of Z.
// Weights come from global memory (L2-resident: 128 KB per head) in fragment order (packed
// once, when the model is built): the 16-byte pieces the 64 lanes of a wave take for one MFMA
// lie back to back, so a load instruction reads 1 KB of whole cache lines.  The hidden
// activations never leave LDS.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace cvr {

constexpr int kMixTM = 64;            // candidates per tile
constexpr int kMixW = 128;            // mixed-token width (16 tokens x 8)
constexpr int kMixHid = 256;          // FFN hidden width
constexpr int kYPitch = kMixW + 4;    // fp32 elements per LDS row (16-byte reads of 16 rows cover all banks)
constexpr int kHPitch = kMixHid + 8;  // bf16 elements per LDS row
constexpr int kMixBlocks = 256;       // one block per CU (the double-buffered tiles take 135 KB of LDS)

// Block b runs on XCD b % 8.  Its slot b / 8 there picks the head (slot % H) and one of
// `groups` tile runs (slot / H); run r = group * 8 + XCD takes tiles r, r + 8 * groups, ...
// The 16 heads of a run sit on one XCD and walk the same tiles together, sharing the token
// rows through its L2 (each head reads and writes 32 bytes of every 512-byte token row).
__global__ __launch_bounds__(512) void token_mix_kernel(const TokenMixParams p, int groups) {
  __shared__ __align__(16) float Ys[2][kMixTM * kYPitch];
  __shared__ __align__(16) bf16 Hs[2][kMixTM * kHPitch];
  __shared__ __align__(16) float bs1[kMixHid];
  __shared__ __align__(16) float bs2[kMixW];
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int h = slot % p.H, run = (slot / p.H) * 8 + xcd, stride = 8 * groups;
  const int tiles = (p.n + kMixTM - 1) / kMixTM;
  if (run >= tiles) return;
  const int ntl = (tiles - run + stride - 1) / stride;  // tiles of this run
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, w = wave & 3;
  const bool first = wave < 4;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  constexpr int T = kMixW / 8;  // 16 tokens of 8 columns per head (checked at launch)
  constexpr int hw = 8;

  // Waves 0-3: piece (w, k, a, lane) = W1[64w + 32a + lane%32][16k + 8(lane/32) .. +7] in
  // wf[2k + a].  Waves 4-7: piece (w, k, lane) = W2[32w + lane%32][16k + 8(lane/32) .. +7] in
  // wf[k].  Either way 16 pieces 64 apart.
  const bf16x8* wsrc = first ? reinterpret_cast<const bf16x8*>(p.W1 + (int64_t)h * p.w1_gstride)
                             : reinterpret_cast<const bf16x8*>(p.W2 + (int64_t)h * p.w2_gstride);
  wsrc += 1024 * w + lane;
  bf16x8 wf[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) wf[i] = wsrc[64 * i];
  if (tid < kMixHid) bs1[tid] = p.b1[(int64_t)h * p.b1_gstride + tid];
  else if (tid < kMixHid + kMixW) bs2[tid - kMixHid] = p.b2[(int64_t)h * p.b2_gstride + tid - kMixHid];

  // Tokens of one tile: row m, element 8t + j <- Y[c0 + m][t][8h + j].  Lanes 2i and 2i + 1
  // load the two 16-byte halves of one token's 32 bytes.
  constexpr int kPer = kMixTM * T * 2 / 512;
  float4 ya[kPer];
  auto load_tile = [&](int tl) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int q = tid + 512 * r, m = q >> 5, t = (q >> 1) & (T - 1), half = q & 1, c = tl * kMixTM + m;
      ya[r] = c < p.n ? *reinterpret_cast<const float4*>(p.Y + ((int64_t)c * T + t) * p.d + h * hw + 4 * half)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stage_tile = [&](float* dst) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int q = tid + 512 * r, m = q >> 5, t = (q >> 1) & (T - 1), half = q & 1;
      *reinterpret_cast<float4*>(&dst[m * kYPitch + t * 8 + 4 * half]) = ya[r];
    }
  };
  load_tile(run);
  stage_tile(Ys[0]);
  __syncthreads();

  for (int s = 0; s <= ntl; ++s) {
    if (s + 1 < ntl) load_tile(run + (s + 1) * stride);  // in flight during this stage
    if (first) {
      if (s < ntl) {
        // 2. hidden^T (units 64w .. 64w+63, 64 candidates) = W1 X^T, K = 128
        const float* X = Ys[s & 1];
        bf16* Hd = Hs[s & 1];
        f32x16 acc[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
#pragma unroll
        for (int k = 0; k < kMixW / 16; ++k) {
          bf16x8 xb[2];
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const float* src = &X[(32 * b + lr) * kYPitch + 16 * k + lk];
            const float4 x0 = *reinterpret_cast<const float4*>(src), x1 = *reinterpret_cast<const float4*>(src + 4);
            xb[b][0] = (bf16)x0.x; xb[b][1] = (bf16)x0.y; xb[b][2] = (bf16)x0.z; xb[b][3] = (bf16)x0.w;
            xb[b][4] = (bf16)x1.x; xb[b][5] = (bf16)x1.y; xb[b][6] = (bf16)x1.z; xb[b][7] = (bf16)x1.w;
          }
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = Lowp<bf16>::mfma32(wf[2 * k + a], xb[b], acc[a][b]);
        }
        // element v of tile (a, b): unit 64w + 32a + 8(v/4) + 4(lane/32) + v%4, candidate 32b + lane%32
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int u = 64 * w + 32 * a + 8 * v4 + (lk >> 1);
            const float4 bb = *reinterpret_cast<const float4*>(&bs1[u]);
            const float bv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              bf16x4 o;
#pragma unroll
              for (int q = 0; q < 4; ++q) o[q] = (bf16)relu_f32(acc[a][b][4 * v4 + q] + bv[q]);
              *reinterpret_cast<bf16x4*>(&Hd[(32 * b + lr) * kHPitch + u]) = o;
            }
          }
      }
    } else if (s >= 1) {
      // 3. F^T (outputs 32w .. 32w+31, 64 candidates) = W2 hidden^T, K = 256; revert + residual
      const float* X = Ys[(s - 1) & 1];
      const bf16* Hd = Hs[(s - 1) & 1];
      const int c0 = (run + (s - 1) * stride) * kMixTM;
      f32x16 acc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
#pragma unroll
      for (int k = 0; k < kMixHid / 16; ++k) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const bf16x8 hb = *reinterpret_cast<const bf16x8*>(&Hd[(32 * b + lr) * kHPitch + 16 * k + lk]);
          acc[b] = Lowp<bf16>::mfma32(wf[k], hb, acc[b]);
        }
      }
      // element v of tile b: output 32w + 8(v/4) + 4(lane/32) + v%4 = 8t + j, candidate 32b + lane%32
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int o = 32 * w + 8 * v4 + (lk >> 1);
        const int t = o / hw, j = o % hw;
        const float4 bb = *reinterpret_cast<const float4*>(&bs2[o]);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int c = c0 + 32 * b + lr;
          if (c >= p.n) continue;
          const float4 y = *reinterpret_cast<const float4*>(&X[(32 * b + lr) * kYPitch + o]);
          float4 z;
          z.x = y.x + (acc[b][4 * v4 + 0] + bb.x);
          z.y = y.y + (acc[b][4 * v4 + 1] + bb.y);
          z.z = y.z + (acc[b][4 * v4 + 2] + bb.z);
          z.w = y.w + (acc[b][4 * v4 + 3] + bb.w);
          const int64_t zo = ((int64_t)c * T + t) * p.d + h * hw + j;
          if (p.Zb) {  // rounded as the next Linear would round it on loading
            bf16x4 zb;
            zb[0] = (bf16)z.x; zb[1] = (bf16)z.y; zb[2] = (bf16)z.z; zb[3] = (bf16)z.w;
            *reinterpret_cast<bf16x4*>(p.Zb + zo) = zb;
          } else {
            *reinterpret_cast<float4*>(p.Z + zo) = z;
          }
        }
      }
    }
    if (s == ntl) break;
    __syncthreads();  // hidden tile s handed over; tile s - 1's token buffer is free
    if (s + 1 < ntl) {
      stage_tile(Ys[(s + 1) & 1]);
      __syncthreads();
    }
  }
}

__global__ void mix_pack_kernel(const float* __restrict__ src, bf16* __restrict__ dst, int which) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;  // 16-byte piece of the packed matrix
  if (g >= kMixW * kMixHid / 8) return;
  const int lane = g & 63, lr = lane & 31, lk = (lane >> 5) * 8, w = g >> 10;
  int row, col, ld;
  if (which == 1) {  // g = ((w * 8 + k) * 2 + a) * 64 + lane
    row = 64 * w + 32 * ((g >> 6) & 1) + lr;
    col = 16 * ((g >> 7) & 7) + lk;
    ld = kMixW;
  } else {           // g = (w * 16 + k) * 64 + lane
    row = 32 * w + lr;
    col = 16 * ((g >> 6) & 15) + lk;
    ld = kMixHid;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[8 * g + j] = Lowp<bf16>::from_f32(src[row * ld + col + j]);
}

hipError_t launch_mix_pack(const float* src, void* dst, int which, hipStream_t st) {
  if (which != 1 && which != 2) return hipErrorInvalidValue;
  launch_k(mix_pack_kernel, dim3(kMixW * kMixHid / 8 / 256), dim3(256), 0, st, src, (bf16*)dst, which);
  return hipGetLastError();
}

bool token_mix_supported(int32_t T, int32_t d, int32_t H, int32_t hidden) {
  return d / H == 8 && d % H == 0 && T * 8 == kMixW && hidden == kMixHid;
}

hipError_t launch_token_mix(const TokenMixParams& p, hipStream_t st) {
  if (p.n <= 0) return hipSuccess;
  if (!token_mix_supported(p.T, p.d, p.H, kMixHid)) return hipErrorInvalidValue;
  const int tiles = (p.n + kMixTM - 1) / kMixTM;
  int groups = kMixBlocks / (8 * p.H);
  groups = std::max(1, std::min(groups, (tiles + 7) / 8));
  launch_k(token_mix_kernel, dim3(8 * groups * p.H), dim3(512), 0, st, p, groups);
  return hipGetLastError();
}

}  // namespace cvr
