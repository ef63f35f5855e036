// Batch padding for graph replay per batch bucket (CVR article section 3.4.4: the serving path
// captures the stable launch sequence once per batch size bucket and replays them).
//
// A captured scoring graph runs at its bucket's sizes.  Before each replay bucket_pad_kernel
// copies the caller's batch into the bucket's staging arrays and pads it: the spare requests
// own no bags and no sequence positions, the spare candidates (at least one, all in the last
// request) own empty bags, and the spare id and position capacity belongs to no bag and no
// sequence, so the padding adds no gather, sequence or attention work.  The sequence ids are not
// copied: the graph's sequence encoder reads the caller's array through the header.  A
// candidate's score depends only on its own bags and its request's bags and sequences, so the
// padding changes no score of the caller's candidates.  The graph ends with bucket_copy_out, which copies the
// caller's scores out of the bucket-sized score buffer to the destination the pad kernel wrote
// into the header.
//
// The kernel only copies and reshapes; it raises no error itself.  Where padding would hide a
// malformed batch -- a last candidate offset other than n_candidates, a last bag offset other
// than n_ids, a sequence offset outside [0, n_positions] -- it writes -1 into the padded offsets,
// which the expand kernel of the replayed graph reports as malformed.
#include "device_common.h"
#include "kernels.h"

namespace cvr {

__global__ __launch_bounds__(256) void bucket_pad_kernel(const BucketPadParams p) {
  const int64_t n_co = (int64_t)p.Rb + 1;
  const int64_t n_bo = p.total_bags_b + 1;
  const int64_t n_so = (int64_t)p.S * (p.Rb + 1);
  const int64_t total = n_co + n_bo + p.n_ids + n_so;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    p.hdr->count = (int64_t)p.n * p.tasks;
    p.hdr->out = p.out;
    p.hdr->seq_ids = p.sid;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t j = i;
    if (j < n_co) {
      int32_t v;
      if (j <= p.R) v = p.co[j];
      else if (j < p.Rb) v = p.n;
      else v = p.co[p.R] == p.n ? p.nb : -1;  // the last spare request owns candidates n .. nb-1
      p.co_b[j] = v;
      continue;
    }
    j -= n_co;
    if (j < n_bo) {
      int32_t v;
      if (j == p.total_bags_b) {
        v = p.bo[p.total_bags] == p.n_ids ? (int32_t)p.n_ids : -1;
      } else {
        int f = 0;
        while (f + 1 < p.nf && p.base_b[f + 1] <= j) ++f;
        const int64_t local = j - p.base_b[f];
        const int64_t nbf = p.base[f + 1] - p.base[f];
        v = p.bo[p.base[f] + (local <= nbf ? local : nbf)];  // spare bags are empty
      }
      p.bo_b[j] = v;
      continue;
    }
    j -= n_bo;
    if (j < p.n_ids) {
      p.ids_bk[j] = p.ids[j];
      continue;
    }
    j -= p.n_ids;
    // Sequence offsets.  Every value written is -1 or inside [0, n_positions] of the caller's
    // batch, so the sequence encoder, reading the caller's seq_ids in place, stays inside them.
    const int s = (int)(j / (p.Rb + 1));
    const int r = (int)(j % (p.Rb + 1));
    int32_t v = p.so[(int64_t)s * (p.R + 1) + (r <= p.R ? r : p.R)];  // spare requests: empty sequences
    if (v < 0 || v > p.P) v = -1;
    p.so_b[j] = v;
  }
}

static void pad_grid(const BucketPadParams& p, dim3& grid, dim3& block) {
  // sized for the bucket, so that the same launch shape serves every batch of the bucket
  const int64_t cap = (int64_t)p.Rb + 1 + p.total_bags_b + 1 + p.ids_b + (int64_t)p.S * (p.Rb + 1);
  int64_t blocks = (cap + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  grid = dim3((unsigned)blocks);
  block = dim3(256);
}

hipError_t launch_bucket_pad(const BucketPadParams& p, hipStream_t st) {
  dim3 grid, block;
  pad_grid(p, grid, block);
  launch_k(bucket_pad_kernel, grid, block, 0, st, p);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void bucket_copy_out_kernel(const BucketHeader* __restrict__ hdr,
                                                              const float* __restrict__ src, int64_t cap) {
  int64_t count = hdr->count;
  count = count < cap ? count : cap;
  float* dst = hdr->out;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_bucket_copy_out(const BucketHeader* hdr, const float* src, int64_t cap, hipStream_t st) {
  int64_t blocks = (cap + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  launch_k(bucket_copy_out_kernel, dim3((unsigned)blocks), dim3(256), 0, st, hdr, src, cap);
  return hipGetLastError();
}

}  // namespace cvr
