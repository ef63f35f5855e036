// Launch interfaces of the libcvr kernels (host side).  Internal to the library.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cvr {

// ---------------------------------------------------------------- kernel launches
// Every kernel goes through launch_k.  When the calling thread has armed a pair of timing
// events (launch_timing), the launch carries them in its dispatch: the begin event is
// stamped when the first kernel of the bracket starts and the end event when the last one
// ends, so the measured time is the kernels' own, without host-side event packets in between.
// Arguments are converted to the kernel's parameter types before they are packed; callers
// read the launch status with hipGetLastError().
struct LaunchTiming {
  hipEvent_t begin = nullptr, end = nullptr;
  int launched = 0;
};
LaunchTiming& launch_timing();
template <typename... KArgs, typename... Args>
inline void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                     Args&&... args) {
  LaunchTiming& t = launch_timing();
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, t.launched == 0 ? t.begin : nullptr, t.end, 0,
                        static_cast<KArgs>(args)...);
  if (t.begin) t.launched++;
}

// Device error flag bits (OR-ed into the workspace's status word).
enum : int32_t {
  ERRF_CAND_OFFSETS = 1,
  ERRF_BAG_OFFSETS = 2,
  ERRF_ID_RANGE = 4,
  ERRF_SEQ_OFFSETS = 8,
  ERRF_SEQ_ID_RANGE = 16,
};

constexpr int kMaxGatherFeatures = 32;
constexpr int kSeqChunk = 32;  // positions per SwiGLU work item (never spanning two sequences)
constexpr int kMaxASegments = 4;

// ---------------------------------------------------------------- expand (A0/B0)
struct ExpandParams {
  const int32_t* cand_offsets;  // [R+1]
  int32_t R;
  int32_t n;
  const int32_t* bag_offsets;   // [total_bags+1]
  int64_t total_bags;
  int64_t n_ids;
  const int32_t* seq_offsets;   // [S][R+1] or null
  int32_t S;
  int64_t n_positions;
  int32_t* cand_req;            // [n] out
  int32_t* flag;                // status word: set to zero by block 0 (later kernels of the call raise into it)
  int32_t* block_err;           // [blocks] out: each block's own check results (0 or ERRF_ bits)
  int32_t ids_capacity;         // 1: n_ids is a capacity, the last bag may end before it (bucket replay)
};
// Blocks of the expand launch for these sizes (one thread per index, 1024 per block).
int64_t expand_blocks(int64_t n, int64_t total_bags, int64_t R, int64_t S);
// blocks: expand_blocks() of the batch (the block_err words the status read covers).
hipError_t launch_expand(const ExpandParams& p, int64_t blocks, hipStream_t st);

// The sequence chunk plan (chunk_plan.h): segment chunk offsets [S*R+1] and chunk descriptors.
struct PlanParams {
  const int32_t* seq_offsets;   // [S][R+1]
  int32_t R, S;
  int64_t n_positions;
  int32_t max_chunks;           // n_positions / 32 + S * R: what the workspace holds
  int32_t* chunk_off;           // [S*R+1] out
  int2* desc;                   // [max_chunks] out
};
constexpr int kPlanMaxSegs = 16000;  // segments whose offset table fits (with the rest) in 64 KB of LDS
int64_t chunk_plan_blocks(int64_t max_chunks);  // about two chunks per thread, at most 256 blocks
// The batch expansion and the chunk plan in one launch (the expand blocks first, then
// chunk_plan_blocks plan blocks); needs S * R <= kPlanMaxSegs.
hipError_t launch_front(const ExpandParams& p, int64_t expand_blocks, const PlanParams& plan, hipStream_t st);
// Whether the CVR path makes its chunk plan in the expand launch (the table fits LDS).
inline bool seq_plan_in_front(int64_t S, int64_t R) { return S * R <= kPlanMaxSegs; }

// ---------------------------------------------------------------- graph replay per batch bucket
// Written by bucket_pad_kernel before each replay, read by the replayed graph's last kernel.
struct BucketHeader {
  int64_t count;           // scores to copy out: n_candidates * n_tasks of the caller's batch
  float* out;              // the caller's out_scores
  const int32_t* seq_ids;  // the caller's seq_ids, read in place by the sequence encoder
};
struct BucketPadParams {
  // the caller's batch
  const int32_t* co;            // cand_offsets [R+1]
  const int32_t* bo;            // bag_offsets [total_bags+1]
  const int32_t* ids;           // [n_ids]
  const int32_t* so;            // seq_offsets [S][R+1] (CVR) or null
  const int32_t* sid;           // seq_ids [P][ncols] (CVR) or null
  int32_t R, n;
  int64_t total_bags, n_ids, P;
  int32_t S, ncols;
  // the bucket
  int32_t Rb, nb;
  int64_t total_bags_b, ids_b, Pb;
  int32_t nf;
  int64_t base[kMaxGatherFeatures + 1];         // first bag of each feature, caller's layout
  int64_t base_b[kMaxGatherFeatures + 1];       // first bag of each feature, bucket layout
  // staging arrays of the bucket (workspace)
  int32_t* co_b;
  int32_t* bo_b;
  int32_t* ids_bk;
  int32_t* so_b;
  BucketHeader* hdr;
  float* out;
  int32_t tasks;
};
hipError_t launch_bucket_pad(const BucketPadParams& p, hipStream_t st);
hipError_t launch_bucket_copy_out(const BucketHeader* hdr, const float* src, int64_t cap, hipStream_t st);

// ---------------------------------------------------------------- HBM hot-row cache
// Directory of one table's cache, in caller-owned device memory (see cache_layout):
// header (epoch, queue length, counters), tags [sets][ways] (row held or -1), stamps
// [sets][ways] (batch of last use), first [sets] (earliest missed lookup of the current batch,
// INT32_MAX if none), queue [sets] (sets that missed in the current batch), rows
// [sets * ways][dim] fp32.
constexpr int kMaxCaches = 4;
constexpr int kCacheMaxWays = 16;
enum { CACHE_LOOKUPS = 0, CACHE_HITS, CACHE_MISSES, CACHE_ADMISSIONS, CACHE_EVICTIONS, CACHE_NCOUNTERS };
struct CacheLayout {
  size_t tags, stamps, first, queue, rows, total;  // byte offsets into the state; total bytes
};
CacheLayout cache_layout(int64_t sets, int32_t ways, int32_t dim);
// Each counter is spread over kCacheCounterSlots addresses (block b adds to slot b mod slots)
// so that thousands of blocks do not queue on one atomic; readers sum the slots.
constexpr int kCacheCounterSlots = 64;
struct CacheHeader {
  int32_t epoch;
  int32_t queued;       // sets in the admission queue of the current batch
  int32_t pad_[14];
  unsigned long long counters[CACHE_NCOUNTERS][kCacheCounterSlots];
};
struct GatherCache {
  int32_t* tags;
  int32_t* stamps;
  int32_t* first;
  int32_t* queue;       // [sets]: the sets that missed in the current batch, each once
  float* rows;
  CacheHeader* hdr;
  int32_t sets, ways;
};
hipError_t launch_cache_init(const GatherCache& c, hipStream_t st);
// Starts a batch: every attached cache's epoch advances by one and its queue empties.
hipError_t launch_cache_begin(CacheHeader* const* hdrs, int n, hipStream_t st);
// After the gather: each set that missed admits the row of its earliest missed lookup into
// its least recently used way, copying the row from the host table.
// max_lookups bounds the queue length (the batch's ids) and sizes the grid.
hipError_t launch_cache_admit(const GatherCache& c, const int32_t* ids, int64_t n_ids, const float* host_table,
                              int64_t rows, int32_t dim, int64_t max_lookups, hipStream_t st);

// ---------------------------------------------------------------- gather + mean-pool (A1-A2/B1)
struct GatherFeature {
  const float* table;
  int64_t rows;
  int32_t dim;          // multiple of 4, <= 256
  int32_t nbags;        // bags of this feature in the batch (R or n)
  int64_t bag_base;     // index of its first bag in bag_offsets
  void* out;            // low-precision matrix; row = local bag index
  int32_t ldo;          // elements per output row
  int32_t col;          // first output column
  float* dbg;           // fp32 pooled [nbags][dim] or null
  int32_t block_begin;  // first block of this feature in the launch
  int32_t cache;        // index into GatherParams::cache when the table sits behind an HBM cache, else -1
};
struct GatherParams {
  GatherFeature f[kMaxGatherFeatures];
  GatherCache cache[kMaxCaches];
  int32_t nf;
  int32_t total_blocks;
  const int32_t* bag_offsets;
  const int32_t* ids;
  int64_t n_ids;
  float clamp;
  int32_t lowp;         // 0 fp16, 1 bf16
  int32_t* flag;
};
// Fills block_begin/total_blocks and launches.
hipError_t launch_gather_pool(GatherParams& p, hipStream_t st);

// ---------------------------------------------------------------- GEMM (MFMA)
// C(m, n) = epilogue( sum_k A(m, k) * W(n, k) + bias(n) ) for a group index g.
// A(m, k): K is split into segments; in segment s (k_begin..k_end) with kk = k - k_begin + col0,
//   A(m, k) = seg.ptr[g*seg.gstride + row*seg.ld + (kk/8)*seg.kstride8 + kk%8], row = rowmap ? rowmap[m] : m.
//   A segment flagged f32 holds fp32 values, rounded to the low-precision type as they are loaded
//   (the rounding every Linear input gets).
// W(n, k) = W[g*w_gstride + n*K + k].   C(m, n) at C[g*c_gstride + m*ldc + (n/8)*c_nstride8 + n%8];
// the optional residual R uses the same addressing as C.
struct ASeg {
  const void* ptr;
  const int32_t* rowmap;
  int64_t ld;
  int64_t gstride;
  int32_t k_end;
  int32_t kstride8;
  int32_t col0;
  int32_t f32;          // 1: source is fp32
};
struct GemmParams {
  int32_t M, N, K;
  int32_t groups;
  int32_t nseg;
  ASeg seg[kMaxASegments];
  const void* W;
  int64_t w_gstride;
  const float* bias;
  int64_t bias_gstride;
  void* C;
  int64_t ldc;
  int64_t c_gstride;
  int32_t c_nstride8;
  const void* R;        // residual (same addressing as C) or null
  const int32_t* r_rowmap;  // if set: the residual of row m is row r_rowmap[m] of R, rows r_ld apart
  int64_t r_ld;
  int32_t relu;
  int32_t relu_end;     // with relu: only columns n < relu_end (0: all columns)
  int32_t out_f32;      // 1: C is fp32, else the low-precision type
  int32_t r_f32;        // 1: R is fp32, else the low-precision type
  // Output-layer fusion (wide kernel only, see gemm_fuses_output): when ow is set, C is not
  // written; for every row m and every 64-column group c, opart[c * opart_ld + m] receives the
  // sum over the group's columns n, in a fixed order, of y[m][n] * ow[n] in fp32, where y is
  // the activation C would have held (bias, ReLU, rounded to the low-precision type).
  const void* ow;
  float* opart;
  int64_t opart_ld;
  // 1: when N <= 128, one 64 x 128 tile covers a group's whole width, so each group reads its
  // A rows once (pays when A is shared and cache-resident, e.g. many candidates per request)
  int32_t full_n;
  // With an fp32 output (small-tile kernel, one group): if set, every output element is also
  // written here rounded to the low-precision type, row m at C2 + m * ldc2 -- the input a later
  // Linear would round it to on loading, at half the bytes.
  void* C2;
  int64_t ldc2;
};
hipError_t launch_gemm(const GemmParams& p, int lowp, hipStream_t st);
// True when launch_gemm runs p on the wide kernel, which can take the output-layer fusion.
bool gemm_fuses_output(const GemmParams& p);
constexpr int kOutGroup = 64;  // columns per output-layer partial

// ---------------------------------------------------------------- DLRM output (A4)
// z[m] = sum_k H[m][k] * w[k] + b  (fp32 accumulation), out[m] = sigmoid(z[m]).
hipError_t launch_dlrm_output(const void* H, int32_t M, int32_t K, const void* w, const float* b,
                              float* logits, float* out, int lowp, hipStream_t st);
// The same from the partials of a fused last hidden layer: z[m] = sum over c = 0..parts-1, in
// order, of part[c * ld + m], plus b; out[m] = sigmoid(z[m]).
hipError_t launch_dlrm_logit(const float* part, int32_t parts, int64_t ld, int32_t M, const float* b, float* logits,
                             float* out, hipStream_t st);

// ---------------------------------------------------------------- CVR sequences (B3-B5)
constexpr int kMaxSeqCols = 8;
constexpr int kMaxTasks = 8;
constexpr int kMaxExperts = 8;

// Chunk table: chunk_off[g] = number of kSeqChunk-position chunks before segment g = s*R + r.
// and one descriptor per chunk (first position; segment << 8 | positions).
hipError_t launch_chunk_table(const int32_t* seq_offsets, int R, int S, int64_t n_positions, int32_t* chunk_off,
                              int2* desc, hipStream_t st);

struct SwigluParams {
  const int32_t* seq_offsets;   // [S][R+1]
  int32_t R, S;
  int64_t n_positions;
  const int32_t* seq_ids;       // [n_positions][ncols]
  const int32_t* const* seq_ids_ref;  // if set, seq_ids is read from here at run time (bucket replay)
  int32_t ncols;
  int32_t col_off[kMaxSeqCols]; // first column of each sequence column in the 128-wide token
  int32_t col_dim[kMaxSeqCols];
  int64_t col_rows[kMaxSeqCols];
  const float* col_table[kMaxSeqCols];
  const int32_t* chunk_off;     // [S*R+1]
  const int2* desc;             // [chunks]
  int32_t max_chunks;           // chunks the workspace holds: n_positions / 32 + S * R
  const __bf16* Wgu;            // per sequence [2*256][128]: gate rows then up rows
  int64_t wgu_gstride;
  const float* bgu;             // per sequence [2*256]
  int64_t bgu_gstride;
  const __bf16* Wd;             // per sequence [128][256]
  int64_t wd_gstride;
  const float* bd;              // per sequence [128]
  int64_t bd_gstride;
  float clamp;
  __bf16* H;                    // [n_positions][128]
  float* part;                  // [chunks][128] column sums
  int32_t* flag;
  int32_t nt;                   // 1: H and the partials leave as nontemporal stores (seq_states_stream)
};
hipError_t launch_swiglu(const SwigluParams& p, int max_chunks, hipStream_t st);
// Encoded states that outsize the last-level cache (256 MB on MI355X) are written, and read by the
// pool and the per-candidate attention of the second and later layers, with nontemporal hints:
// they cannot stay cached between the launches anyway, and a streaming read runs at about
// 7.0 TB/s with the hint against 6.3 without.  Smaller ones are kept cacheable, since the
// attention then finds them in that cache.
constexpr int64_t kStateStreamBytes = 256LL << 20;
inline bool seq_states_stream(int64_t n_positions) { return n_positions * 128 * 2 >= kStateStreamBytes; }
// pool_bf: if set, the pools are also written there rounded to bf16 (the query Linear's input).
hipError_t launch_seq_pool(const float* part, const int32_t* chunk_off, const int32_t* seq_offsets, int R, int S,
                           int64_t n_positions, int32_t max_chunks, float* pool, __bf16* pool_bf, bool nt,
                           hipStream_t st);

// ---------------------------------------------------------------- attention (B7)
struct AttnParams {
  const __bf16* H;              // [n_positions][128]
  const int32_t* seq_offsets;   // [S][R+1]
  int32_t R, S;
  int64_t n_positions;
  const float* q;               // [S][n][128]
  const int32_t* cand_req;      // [n]
  int32_t n;
  float inv_tau;
  float* Y;                     // [n][T][128]: writes token N+s
  int32_t T, N;
  int32_t mq;                   // 1: MFMA products per request (attention_mq_kernel), 0: per candidate
  int32_t nt;                   // per candidate: 1 reads H with nontemporal loads (seq_states_stream)
};
hipError_t launch_attention(const AttnParams& p, hipStream_t st);
// Default choice of the MFMA form: requests carry 16 or more candidates on average.
bool attention_many_candidates(int32_t n, int32_t R);

// ---------------------------------------------------------------- fused token mixer (B8)
// Z = Y + Revert(FFN_h(Mix_h(Y))) for all heads h in one launch (16 tokens x 128, heads of 8,
// FFN 128 -> 256 -> 128); other shapes take the two grouped GEMMs.
struct TokenMixParams {
  const float* Y;               // [n][T][d] fp32
  float* Z;                     // [n][T][d] fp32
  __bf16* Zb;                   // if set: Z is written here as bf16 instead (Z unused)
  int32_t n, T, d, H;
  const __bf16* W1;             // head h: W1 + h*w1_gstride, [256][T*8] packed by launch_mix_pack
  int64_t w1_gstride;
  const float* b1;
  int64_t b1_gstride;
  const __bf16* W2;             // head h: W2 + h*w2_gstride, [T*8][256] packed by launch_mix_pack
  int64_t w2_gstride;
  const float* b2;
  int64_t b2_gstride;
};
bool token_mix_supported(int32_t T, int32_t d, int32_t H, int32_t hidden);
hipError_t launch_token_mix(const TokenMixParams& p, hipStream_t st);
// One head's first (which = 1, [256][128]) or second (which = 2, [128][256]) mixer Linear,
// fp32 row-major, rounded to bf16 and stored in the order the fused mixer's waves read their
// MFMA operands: every 16-byte piece a lane loads sits next to its neighbours' pieces.
hipError_t launch_mix_pack(const float* src, void* dst, int which, hipStream_t st);

// ---------------------------------------------------------------- EPNet (before B2)
// e' = bf16(2 sigmoid(g) * e) over the D model-input columns of n candidates; e is read in place
// from the request-side matrix (through cand_req) or the item-side matrix, run by run.
struct EpnetParams {
  int32_t n, D;
  const float* g;               // [n][D] gate pre-activations
  const __bf16* x_req;
  const __bf16* x_item;
  int64_t ld_req, ld_item;
  const int32_t* cand_req;
  int32_t nruns;
  int32_t run_k0[kMaxASegments];    // first model-input column of each run of same-side features
  int32_t run_col0[kMaxASegments];  // its first column in its side's matrix
  int32_t run_item[kMaxASegments];  // 1: item-side run
  __bf16* out;                  // [n][D]
};
hipError_t launch_epnet_apply(const EpnetParams& p, hipStream_t st);

// ---------------------------------------------------------------- PLE gates and heads (B10-B11)
struct PleGateParams {
  // Row c of the expert GEMM output (row stride ld): the E expert outputs [E][edim] (after
  // ReLU), then the gate logits of every task, task k's at columns gate0 + goff[k] ...
  const float* experts;
  int64_t ld;
  int32_t n, E, K, edim, gate0;
  int32_t goff[kMaxTasks];
  int32_t emask[kMaxTasks];     // task k mixes expert e iff bit e is set
  __bf16* task_in;              // [K][n][edim]
};
hipError_t launch_ple_gate(const PleGateParams& p, hipStream_t st);

struct HeadOutParams {
  const __bf16* U;              // [K][n][hdim]
  int32_t n, K, hdim;
  const __bf16* w2;             // task k: w2 + k*w2_stride, [hdim]
  int64_t w2_stride;
  const float* b2[kMaxTasks];
  float* logits;                // [n][K]
  float* out;                   // [n][K]
};
hipError_t launch_head_out(const HeadOutParams& p, hipStream_t st);

// The gate mixtures, the heads' first Linear + ReLU and their output Linear + sigmoid in one
// launch (32 candidates per block, the intermediate rows in LDS); the values of the three
// separate kernels.  Needs edim and hdim multiples of 32 and at most kHeadsMaxDim, at most
// kHeadsMaxExperts experts and kHeadsMaxTasks tasks.
constexpr int kHeadsMaxDim = 256;
constexpr int kHeadsMaxExperts = 4;
constexpr int kHeadsMaxTasks = 4;
struct HeadsParams {
  PleGateParams g;              // task_in unused
  const __bf16* W1;             // task k: W1 + k*w1_stride, [hdim][edim]
  int64_t w1_stride;
  const float* b1;              // task k: b1 + k*b1_stride, [hdim]
  int64_t b1_stride;
  int32_t hdim;
  const __bf16* w2;             // task k: w2 + k*w2_stride, [hdim]
  int64_t w2_stride;
  const float* b2[kMaxTasks];
  float* logits;                // [n][K]
  float* out;                   // [n][K]
};
bool heads_fusable(int32_t edim, int32_t hdim, int32_t n_experts, int32_t n_tasks);
hipError_t launch_heads(const HeadsParams& p, hipStream_t st);

// ---------------------------------------------------------------- fill (input generator)
hipError_t launch_fill_table(float* t, int64_t total, uint64_t seed, double step, hipStream_t st);

// ---------------------------------------------------------------- weight packing
// fp32 -> low precision, elementwise (n elements).
hipError_t launch_convert(const float* src, void* dst, int64_t n, int lowp, hipStream_t st);

}  // namespace cvr
