// EPNet scaling of the non-sequence embedding (optional step before B2).
//
// The CVR article (section 3.2.1) obtains the non-sequence embedding through EPNet, which
// models several scenarios.  Taken as PEPNet defines it (Chang et al., KDD 2023): a gate unit
// maps the scenario features' embedding, concatenated with the general embedding, to a
// per-element scale delta = 2 * sigmoid(g), g = W2 ReLU(W1 [e_domain, e] + b1) + b2, and the
// general embedding is multiplied by it.  The two Linears run as GEMMs (the first reads the
// scenario columns and every input run in place, request-side columns through the
// candidate -> request map); this kernel forms delta from g and writes the scaled input,
// rounded to bf16, as the tokenizer's A operand.
#include "device_common.h"
#include "kernels.h"

namespace cvr {

// One thread per 8 consecutive input columns of one candidate (runs are multiples of 32 wide,
// so 8 columns never straddle two runs): 32 bytes of g, 16 bytes of e, 16 bytes out.
__global__ __launch_bounds__(256) void epnet_apply_kernel(const EpnetParams p) {
  const int per_row = p.D / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.n * per_row) return;
  const int64_t c = idx / per_row;
  const int j0 = (int)(idx % per_row) * 8;
  int r = 0;
#pragma unroll
  for (int k = 1; k < kMaxASegments; ++k)
    if (k < p.nruns && j0 >= p.run_k0[k]) r = k;
  const int col = p.run_col0[r] + (j0 - p.run_k0[r]);
  const bf16* src = p.run_item[r] ? p.x_item + c * p.ld_item + col : p.x_req + (int64_t)p.cand_req[c] * p.ld_req + col;
  const bf16x8 e = *reinterpret_cast<const bf16x8*>(src);
  const float4 g0 = *reinterpret_cast<const float4*>(p.g + c * p.D + j0);
  const float4 g1 = *reinterpret_cast<const float4*>(p.g + c * p.D + j0 + 4);
  const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float delta = 2.0f / (1.0f + expf(-g[i]));  // exp(-g) = inf for g << 0: delta = 0
    o[i] = (bf16)(delta * (float)e[i]);
  }
  *reinterpret_cast<bf16x8*>(p.out + c * p.D + j0) = o;
}

hipError_t launch_epnet_apply(const EpnetParams& p, hipStream_t st) {
  const int64_t work = (int64_t)p.n * (p.D / 8);
  if (work <= 0) return hipSuccess;
  launch_k(epnet_apply_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace cvr
