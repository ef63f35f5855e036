/*
 * cvr.h — C ABI of the MI355X candidate-scoring library (libcvr.so).
 *
 * What the library computes.  For every candidate item of every ad request it
 * evaluates one forward pass of a ranking model and writes fp32 probabilities:
 *
 *   - DLRM-style model ("GPU inference optimisation for ad CTR models", the
 *     CTR article): mean-pooled fp32 embeddings, clamp to +-bound, cast to
 *     fp16, an MLP of fp16 Linear+ReLU layers over all candidates with shared
 *     weights (sections 三 and 四), a final 1-unit Linear and an fp32 sigmoid.
 *   - HyFormer-style CVR model (the iQIYI CVR article, section 3.2): the same
 *     pooled embeddings cast to bf16 and projected into N tokens; three
 *     behaviour sequences encoded position by position with SwiGLU; per
 *     sequence one query from the tokens and the sequence's mean pool,
 *     cross-attending to the encoded sequence with a temperature-scaled
 *     softmax (Query Decoding); a Split -> Mixing -> Reverting token mixer
 *     with residual over the N+3 tokens (Query Boosting), stacked n_layers
 *     times; PLE experts with per-task gates and two-layer heads, each
 *     ending in an fp32 sigmoid (section 3.2.4).
 *
 * Precision plan (CTR article section 三; CVR article section 3.4.3): tables
 * and pooling fp32; every Linear weight matrix and every Linear input in fp16
 * (DLRM) or bf16 (CVR), rounded to nearest-even -- in the DLRM model that is
 * every hidden activation; in the CVR model also the encoded sequence states,
 * while its token matrix, queries, attention outputs and expert outputs stay
 * fp32; accumulation, biases, activation functions, softmax, pooling sums and
 * residual adds in fp32; outputs fp32.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP global memory) unless a
 *     comment says "host".  Integer tensors are int32, little-endian.
 *   - The library never allocates device memory.  Weight arena and workspace
 *     are caller-owned; their sizes come from cvr_weight_arena_bytes and
 *     cvr_workspace_bytes.  Tables are borrowed, never copied.
 *   - All device work is enqueued on the caller's stream (a hipStream_t
 *     passed as void*; NULL is the default stream).  Nothing synchronises
 *     except cvr_create (which finishes packing weights before it returns),
 *     cvr_sync_status and cvr_timing_end.
 *   - Every entry point returns a cvr_status; no C++ exception crosses the
 *     ABI.  cvr_last_error gives a message for the last failing call on a
 *     handle (or, with a NULL handle, the last failing call of the thread).
 *   - A handle is not thread-safe; concurrent scoring needs one handle (or
 *     at least one workspace and stream) per thread.
 */
#ifndef CVR_H
#define CVR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cvr_model* cvr_handle;

typedef enum {
  CVR_OK = 0,
  CVR_ERR_ARG = 1,          /* null/misaligned pointer, bad size or count */
  CVR_ERR_SPEC = 2,         /* spec inconsistent, weight missing or misshapen */
  CVR_ERR_RANGE = 3,        /* device found an id/offset out of range (reported by cvr_sync_status) */
  CVR_ERR_WORKSPACE = 4,    /* workspace or arena too small for the call */
  CVR_ERR_HIP = 5,          /* a HIP runtime call failed */
  CVR_ERR_UNSUPPORTED = 6   /* valid spec outside what the kernels implement */
} cvr_status;

enum { CVR_MODEL_DLRM = 0, CVR_MODEL_HYFORMER = 1 };
enum { CVR_SIDE_USER = 0, CVR_SIDE_ITEM = 1, CVR_SIDE_CONTEXT = 2 };
enum { CVR_LOWP_FP16 = 0, CVR_LOWP_BF16 = 1 };

/* One embedding table: fp32, row-major [rows][dim], device memory, BORROWED
 * until cvr_destroy.  dim must be a multiple of 4 (16-byte rows quarters). */
typedef struct {
  const float* data;
  int64_t rows;
  int32_t dim;
} cvr_table;

/* One sparse feature: which table its ids index and whose bag it is.
 * side = USER or CONTEXT: one bag per request; side = ITEM: one bag per
 * candidate (CVR article section 3.4.5: user and item features batched
 * separately, linked by the request). */
typedef struct {
  int32_t table;
  int32_t side;
} cvr_feature;

/* Fixed model information (CVR article section 3.3: what stays fixed between
 * requests is configuration; what varies per request is tensor input).
 * The model input of a candidate is the concat, over features in this order,
 * of each feature's pooled bag.  Fields marked (CVR) are ignored for DLRM. */
typedef struct {
  int32_t model;            /* CVR_MODEL_DLRM or CVR_MODEL_HYFORMER */
  int32_t lowp;             /* DLRM: CVR_LOWP_FP16 or CVR_LOWP_BF16; CVR: CVR_LOWP_BF16 only
                               (CVR_ERR_UNSUPPORTED otherwise) */
  float clamp;              /* clamp bound after pooling (CTR article section 三: 10) */
  int32_t n_features;
  const cvr_feature* features;   /* host array [n_features] */
  int32_t n_hidden;              /* DLRM: hidden Linear+ReLU layers (3-5 in the CTR article) */
  const int32_t* hidden;         /* host array [n_hidden]: widths (1024) */
  /* (CVR) */
  int32_t d;                /* token width (128) */
  int32_t n_tokens;         /* N non-sequence tokens (13) */
  int32_t n_layers;         /* stacked interaction layers (1 or 2) */
  int32_t n_seq;            /* behaviour sequences = queries (3) */
  int32_t n_seq_cols;       /* columns per sequence position (4: item, action, time bucket, side) */
  const int32_t* seq_tables;/* host array [n_seq_cols]: table of each column; dims must sum to d */
  int32_t swiglu_hidden;    /* SwiGLU hidden width (256) */
  float tau;                /* attention temperature (2*sqrt(d)) */
  int32_t mixer_heads;      /* token-mixer split count (16) */
  int32_t mixer_hidden;     /* per-mixed-token FFN hidden width (256) */
  int32_t n_experts;        /* PLE experts (3) */
  int32_t expert_dim;       /* expert width (256) */
  int32_t n_tasks;          /* scenarios / heads (2) */
  int32_t head_hidden;      /* head hidden width (128) */
  /* (CVR) Which experts each task's gate mixes: task_experts[k * n_experts + e]
   * is 1 if task k mixes expert e, else 0; every task needs at least one.
   * NULL: every task mixes every expert (shared experts only, MMoE-style).
   * With 3 experts and 2 tasks, {1,0,1, 0,1,1} is PLE with one task-specific
   * expert per task plus one shared expert (CVR article section 3.2.4).  Gate
   * k's Linear has one output per expert it mixes, in expert order. */
  const int32_t* task_experts;
  /* (CVR) EPNet: 0 (off), or the hidden width (a multiple of 32) of the gate unit that scales
   * the non-sequence embedding before tokenization (CVR article section 3.2.1; read as
   * PEPNet's gate: e' = e * 2 sigmoid(W2 ReLU(W1 [e_domain, e] + b1) + b2), e_domain the
   * context-side features' columns).  Weights epnet.fc1.{weight,bias} [hidden][D_domain + D],
   * epnet.fc2.{weight,bias} [D][hidden].  Needs at least one context-side feature. */
  int32_t epnet_hidden;
} cvr_spec;

/* One dense parameter, fp32, device memory, read only during cvr_create.
 * Linear weights are [out][in] row-major.  Names:
 *   DLRM: mlp.<i>.weight / mlp.<i>.bias for i = 0..n_hidden (the last is the 1-unit output).
 *   CVR:  tok.{weight,bias}; seq.<s>.{gate,up,down}.{weight,bias};
 *         layer.<l>.query.<s>.{weight,bias}; layer.<l>.mix.<h>.{fc1,fc2}.{weight,bias};
 *         ple.expert.<e>.{weight,bias}; ple.gate.<k>.{weight,bias};
 *         head.<k>.{fc1,fc2}.{weight,bias}; with EPNet also epnet.{fc1,fc2}.{weight,bias}. */
typedef struct {
  const char* name;         /* host string */
  const float* data;        /* device */
  int64_t numel;
} cvr_weight;

/* One batch of requests in CSR form (all device int32 arrays).
 *   cand_offsets [n_requests+1]: request r owns candidates cand_offsets[r] ..
 *     cand_offsets[r+1]-1; cand_offsets[0] = 0, non-decreasing,
 *     cand_offsets[n_requests] = n_candidates.
 *   bag_offsets [total_bags+1], ids [n_ids]: bags feature-major in spec order;
 *     a user/context feature has n_requests bags (request order), an item
 *     feature n_candidates bags (candidate order); bag_offsets[0] = 0,
 *     non-decreasing, bag_offsets[total_bags] = n_ids; ids are table rows.
 *   (CVR) seq_offsets [n_seq][n_requests+1]: positions of sequence s of
 *     request r are rows seq_offsets[s][r] .. seq_offsets[s][r+1]-1 of
 *     seq_ids; all inside [0, n_positions], and the whole array read as one
 *     list is non-decreasing (within each s, and seq_offsets[s][n_requests] <=
 *     seq_offsets[s+1][0]), so no position belongs to two sequences.
 *     n_seq * n_requests < 2^23.
 *   (CVR) seq_ids [n_positions][n_seq_cols]: table rows of each column.
 * Offsets are per-request metadata passed as tensors (CVR article section
 * 3.3); the caller packs them on the host and copies them in one transfer
 * (section 3.4.1).  Malformed offsets or ids never make the kernels read
 * outside these arrays or the tables: they raise the device error flag. */
typedef struct {
  int32_t n_requests;
  int32_t n_candidates;
  int64_t n_ids;
  int64_t n_positions;
  const int32_t* cand_offsets;
  const int32_t* bag_offsets;
  const int32_t* ids;
  const int32_t* seq_offsets;
  const int32_t* seq_ids;
} cvr_batch;

/* Device bytes needed for the packed weights of a spec (tables give dims;
 * their data pointers are not read). */
cvr_status cvr_weight_arena_bytes(const cvr_spec* spec, const cvr_table* tables, int32_t n_tables,
                                  size_t* bytes);

/* Build a model: validate spec, tables and weights; convert the fp32 weights
 * into the low-precision packed layout inside weight_arena (device memory of
 * at least cvr_weight_arena_bytes, 256-byte aligned, caller-owned, kept alive
 * until cvr_destroy).  Synchronises the stream before returning.  On failure
 * *out is NULL. */
cvr_status cvr_create(const cvr_spec* spec, const cvr_table* tables, int32_t n_tables,
                      const cvr_weight* weights, int32_t n_weights, void* weight_arena,
                      size_t arena_bytes, void* hip_stream, cvr_handle* out);

/* Device bytes of workspace one cvr_score call needs for batches up to the
 * given sizes (max_positions is ignored for DLRM). */
cvr_status cvr_workspace_bytes(cvr_handle h, int32_t max_requests, int32_t max_candidates,
                               int64_t max_ids, int64_t max_positions, size_t* bytes);

/* Score one batch: out_scores[c * n_tasks + k] (device fp32, n_tasks = 1 for
 * DLRM) for every candidate c and task k.  workspace: device, 256-byte
 * aligned, at least cvr_workspace_bytes for this batch's sizes.  Host-side
 * checks return at once; device-side checks are reported by cvr_sync_status.
 * Enqueued on hip_stream; returns without synchronising.
 * DLRM specs run the hidden layers over slices of the candidates, each slice
 * through every layer before the next (at most 128 MB per activation buffer:
 * 65536 candidates at width 1024; CVR_OPT_DLRM_PASS_ROWS sets another slice
 * size).  Scores do not depend on the slicing.  With debug on, one slice
 * covers the batch so that the last hidden layer can be exported whole.  With
 * debug off, a last hidden layer that runs on the wide GEMM kernel also forms
 * the output layer's per-row partial sums over 64-column groups and stores
 * no activations; a small kernel adds the partials in group order, adds the
 * bias and applies the sigmoid (the same values as the separate output
 * kernel up to the order of the fp32 additions). */
cvr_status cvr_score(cvr_handle h, const cvr_batch* batch, void* workspace, size_t ws_bytes,
                     float* out_scores, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): cvr_score without a workspace argument.  The
 * workspace is a fixed array of CVR_NOALLOC_SCRATCH_BYTES in the library's own device memory,
 * one per device, held until the process ends; the call itself allocates nothing.  Batches
 * whose cvr_workspace_bytes exceed it return CVR_ERR_WORKSPACE (64 MiB holds, e.g., a request
 * of 1 user + 500 candidates of either model, or a few thousand DLRM candidates).  Every call
 * on a device shares that device's array: calls that overlap on one device (several streams,
 * threads or models) race and must be serialised by the caller.  cvr_sync_status and
 * cvr_debug_export read the array as they read a workspace, until the next call on the
 * device.  Same results as cvr_score (the same kernels). */
#define CVR_NOALLOC_SCRATCH_BYTES (64u << 20)
cvr_status cvr_score_noalloc(cvr_handle h, const cvr_batch* batch, float* out_scores, void* hip_stream);

/* cvr_score through graph replay per batch bucket (CVR article section 3.4.4:
 * the serving path captures the scoring launches once per batch size bucket
 * and replays them, reusing the same buffers).  Same arguments and result as
 * cvr_score.  The batch's bucket is its four sizes rounded up -- requests + 1
 * and candidates + 1 (one spare of each), ids and positions as they are -- each
 * to the next m * 2^k with 8 <= m <= 16 (sizes below 16 stay exact), so a
 * bucket holds at most 12.5% more than the batch in each size plus the spares.
 * The first call for a bucket (with this workspace, ws_bytes, stream and debug
 * setting) captures one scoring call at the bucket's sizes into a HIP graph;
 * later calls in the bucket replay it without capturing.  Every call first
 * launches one kernel that copies the batch into the bucket's staging arrays
 * in the workspace and pads it with requests, candidates, bags and positions
 * that belong to no caller request (their scores are computed and dropped:
 * the padding costs up to the bucket's extra size in work); the graph ends by
 * copying the caller's scores to out_scores.  Scores equal cvr_score's on the
 * same batch when the bucket's sizes select the same kernels (the kernel
 * choices depend on sizes: CVR_OPT_TOK_SHARE and CVR_OPT_ATTN_MQ fix two of
 * them), else up to the order of fp32 additions.  At most 8 graphs are held
 * per model (least recently used released first); cvr_set_option and
 * cvr_cache_attach release them all.  workspace: at least
 * cvr_graph_workspace_bytes for the batch's sizes (more than cvr_score
 * needs).  hip_stream must be a created stream (CVR_ERR_ARG for the null
 * stream); cvr_timing does not record graph launches.  Host-side checks run on
 * every call; device-side checks are reported by cvr_sync_status as for
 * cvr_score, malformed offsets included (the padding keeps them malformed).
 * After a replay, cvr_debug_export describes the padded batch: per-request
 * and per-candidate rows of the caller's batch first, padding after them.
 * Graphs are released by cvr_destroy. */
cvr_status cvr_score_graph(cvr_handle h, const cvr_batch* batch, void* workspace, size_t ws_bytes,
                           float* out_scores, void* hip_stream);

/* Device bytes of workspace cvr_score_graph needs for batches up to the given
 * sizes (those of their bucket; max_positions is ignored for DLRM). */
cvr_status cvr_graph_workspace_bytes(cvr_handle h, int32_t max_requests, int32_t max_candidates, int64_t max_ids,
                                     int64_t max_positions, size_t* bytes);

/* Graphs held by the model and graphs captured since cvr_create (host values). */
cvr_status cvr_graph_info(cvr_handle h, int64_t* graphs_held, int64_t* captures);

/* Kernel-selection options of a model.  Each has a default that scoring uses unless the option
 * is set; scores do not depend on them beyond the order of fp32 additions (DLRM_PASS_ROWS and
 * STATE_STREAM: not at all).  Setting an option discards a graph captured by cvr_score_graph.  Values:
 *   CVR_OPT_DLRM_PASS_ROWS  DLRM: candidates per MLP pass (each pass through every layer before
 *                           the next).  -1 (default): as many as fill 128 MB per activation
 *                           buffer (65536 at width 1024); 0: one pass; k > 0: k candidates.
 *   CVR_OPT_TOK_SHARE       CVR: tokenizer request-side columns multiplied once per request and
 *                           added to every candidate of the request.  -1 (default): when requests
 *                           average 4 or more candidates; 0: never; 1: whenever the spec allows.
 *   CVR_OPT_ATTN_MQ         CVR: attention of a request's candidates as MFMA products over its
 *                           shared states.  -1 (default): when requests average 16 or more
 *                           candidates; 0: never (one block per candidate); 1: always.
 *   CVR_OPT_DLRM_USER_BLOCK DLRM: the first Linear's request-side columns multiplied once per
 *                           request (U = X_req W_req^T in fp32) and U's row added to every
 *                           candidate's item-side product (CTR article section 四, CVR article
 *                           section 3.4.5).  -1 (default) and 0: off; 1: on (CVR_ERR_UNSUPPORTED
 *                           unless the spec has request-side and item-side features in runs of
 *                           multiples of 32 columns).
 *   CVR_OPT_HEADS_FUSED     CVR: the PLE gate mixture, the heads' two Linears and the sigmoid in
 *                           one launch (CVR article section 3.2.4), with the values of the
 *                           three separate launches.  -1 (default) and 1: fused when expert_dim
 *                           and head_hidden are at most 256, with at most 4 experts and 4 tasks
 *                           (1 beyond that: CVR_ERR_UNSUPPORTED); 0: three launches.
 *   CVR_OPT_STATE_STREAM    CVR: the encoded sequence states (and the encoder's per-chunk pool
 *                           partials) written, and read by the pool and by the per-candidate
 *                           attention of the second and later layers, with nontemporal hints.  A cache policy only: results do
 *                           not depend on it at all.  -1 (default): when the states take 256 MB
 *                           or more (they then outsize the last-level cache); 0: never; 1: always.
 * Unknown options and values outside these ranges return CVR_ERR_ARG. */
enum {
  CVR_OPT_DLRM_PASS_ROWS = 0,
  CVR_OPT_TOK_SHARE = 1,
  CVR_OPT_ATTN_MQ = 2,
  CVR_OPT_DLRM_USER_BLOCK = 3,
  CVR_OPT_HEADS_FUSED = 4,
  CVR_OPT_STATE_STREAM = 5
};
cvr_status cvr_set_option(cvr_handle h, int32_t option, int64_t value);

/* Wait for the stream and report the device error flag of the last
 * cvr_score on that workspace: CVR_ERR_RANGE if an id was outside its table
 * or offsets were malformed (the batch's scores must then be discarded). */
cvr_status cvr_sync_status(cvr_handle h, void* hip_stream);

/* Intermediates kept in the workspace after the last cvr_score, for parity
 * checks.  Copied (device to device, on hip_stream) into dst of dst_bytes;
 * *written gets the byte count.  CVR_DBG_POOLED needs debug != 0 at
 * cvr_set_debug time before the scoring call. */
enum {
  CVR_DBG_CAND_REQ = 0,     /* int32 [n]: request of each candidate */
  CVR_DBG_POOLED = 1,       /* fp32, per feature in spec order: [bags_f][dim_f] pooled means before clamp */
  CVR_DBG_INPUT_REQ = 2,    /* lowp [n_requests][D_req]: clamped, cast request-side inputs */
  CVR_DBG_INPUT_ITEM = 3,   /* lowp [n][D_item]: clamped, cast item-side inputs */
  CVR_DBG_LOGITS = 4,       /* fp32 [n][n_tasks]: pre-sigmoid outputs */
  CVR_DBG_HSEQ = 5,         /* (CVR) bf16 [n_positions][d]: SwiGLU outputs */
  CVR_DBG_SEQ_POOL = 6,     /* (CVR) fp32 [n_seq][n_requests][d]: mean pools */
  CVR_DBG_TOKENS = 7,       /* (CVR) fp32 [n][N+n_seq][d]: last layer's token matrix Z (needs debug != 0 at
                               scoring when the fused token mixer runs: it then writes Z as bf16) */
  CVR_DBG_QUERY = 8,        /* (CVR) fp32 [n_seq][n][d]: last layer's queries */
  CVR_DBG_ATTN = 9,         /* (CVR) fp32 [n][N+n_seq][d]: last layer's token matrix before mixing (attention outputs in rows N..) */
  CVR_DBG_HIDDEN = 10,      /* (DLRM, debug mode) lowp [n][width]: activations of the last hidden
                               layer (outside debug mode that layer may hand per-row partials of
                               the output layer to it instead of storing its activations) */
  CVR_DBG_EPNET = 11        /* (CVR with EPNet) bf16 [n][D]: the scaled model input (tokenizer input) */
};
cvr_status cvr_set_debug(cvr_handle h, int32_t debug);
cvr_status cvr_debug_export(cvr_handle h, int32_t what, void* dst, size_t dst_bytes, size_t* written,
                            void* hip_stream);

/* HBM hot-row cache over a host-resident table (CTR article section 二: hot
 * embeddings in GPU HBM in front of host DRAM, least-recently-used
 * replacement, hit and miss rates monitored).
 *
 * The table's data pointer given to cvr_create points to pinned host memory
 * (hipHostMalloc) or to device memory.  Once a cache is attached, every
 * scoring call looks each id of the features that read the table up in the
 * cache: a hit reads the row from HBM, a miss reads it from the table itself
 * (over the bus for host memory).  Pooled values are the same either way.
 * The cache has `sets` x `ways` entries; row r belongs to set fmix32(r) mod
 * sets (fmix32 = MurmurHash3's 32-bit finaliser).  Time is counted in scoring
 * calls: call t stamps every way it hits with t, and all its lookups see the
 * cache as it was when the call began.  After its lookups, each set that
 * missed admits one row, that of its earliest missed lookup (smallest
 * position in batch.ids), into its least recently used way: an empty way
 * first, then the smallest stamp, ties to the lowest way.  Counters since
 * attach: lookups, hits, misses (lookups = hits + misses; ids outside the
 * table are not counted), admissions, evictions (admissions that replaced a
 * row).
 *
 * cvr_cache_state_bytes: device bytes of one cache's state (directory and
 * rows) for the given shape and the table's dim.
 * cvr_cache_attach: serve `table` (index into cvr_create's tables; it must
 * feed at least one feature and no sequence column) through a cache whose
 * state lives in `state` (device memory of at least cvr_cache_state_bytes,
 * 256-byte aligned, caller-owned, kept alive until cvr_destroy).  1 <= ways <=
 * min(16, dim/4), 1 <= sets, sets * ways < 2^31; at most 4 caches per model;
 * a table takes one cache.  Initialises the state (empty, counters zero) on
 * hip_stream.  Scoring calls enqueued afterwards use it; a graph captured by
 * cvr_score_graph before the attach is discarded.
 * cvr_cache_stats: waits for hip_stream and writes the five counters
 * (lookups, hits, misses, admissions, evictions) to counters[0..4] (host).
 * cvr_cache_export: waits for hip_stream and copies the directory to host
 * arrays of sets * ways int32: tags (row held, -1 if empty) and stamps (call
 * of last use; 0 for a way never filled).
 * Calls that overlap on one model race on its caches. */
cvr_status cvr_cache_state_bytes(int64_t sets, int32_t ways, int32_t dim, size_t* bytes);
cvr_status cvr_cache_attach(cvr_handle h, int32_t table, int64_t sets, int32_t ways, void* state,
                            size_t state_bytes, void* hip_stream);
cvr_status cvr_cache_stats(cvr_handle h, int32_t table, int64_t* counters, void* hip_stream);
cvr_status cvr_cache_export(cvr_handle h, int32_t table, int32_t* tags, int32_t* stamps, void* hip_stream);

/* Per-stage kernel timing with HIP events recorded on the scoring stream.
 * cvr_timing_begin arms up to max_calls subsequent cvr_score calls;
 * stage_mask selects the stages that are timed (bit s for stage s, as
 * numbered by cvr_stage_name; 0 = every stage; a bit past the last stage is
 * CVR_ERR_ARG).  The events ride on the timed stages' kernel dispatches, and
 * such a dispatch costs a few microseconds more than a plain one: timing one
 * stage disturbs a step less than timing all of them.
 * cvr_timing_end waits for them and writes, per stage, the summed
 * milliseconds and the number of kernel launches (0 for stages not timed).
 * Stage names come from cvr_stage_name. */
cvr_status cvr_timing_begin(cvr_handle h, int32_t max_calls, uint32_t stage_mask);
cvr_status cvr_timing_end(cvr_handle h, double* stage_ms, int32_t* stage_launches, int32_t max_stages,
                          int32_t* n_stages, int32_t* n_calls);
const char* cvr_stage_name(cvr_handle h, int32_t stage);

/* Fill a device fp32 table [rows][dim] with synthetic values: element
 * i = row*dim + col is (k - 2^23) * (2*halfwidth / 2^24) in fp64, rounded to
 * fp32, where k is the top 24 bits of the (i+1)-th output of SplitMix64
 * (Steele, Lea & Flood 2014) seeded with seed.  An input generator for tests
 * and benchmarks; not part of scoring. */
cvr_status cvr_fill_table(float* table, int64_t rows, int32_t dim, uint64_t seed, double halfwidth,
                          void* hip_stream);

/* Read-bandwidth probes: the ceilings the streaming kernels are measured
 * against; not part of scoring.  Each block xors what it read into one
 * uint32 of sink (device, >= blocks entries, caller-owned), so no load is
 * dropped; the value means nothing else.  Both enqueue one kernel of
 * `blocks` blocks of 256 threads (1 <= blocks <= 2^20) on hip_stream and
 * return CVR_ERR_ARG on a null pointer or a size outside the stated range.
 * nontemporal: 0 loads plainly, 1 with the nontemporal hint (faster for data
 * that cannot stay cached, slower where the last-level cache holds part of
 * it); other values are CVR_ERR_ARG.
 * cvr_probe_stream_read: reads `bytes` (a multiple of 16) of device memory
 *   at src (16-byte aligned) once, front to back, 16 bytes per lane and
 *   eight loads in flight per lane -- the access pattern of the cross-
 *   attention over encoded states (CVR article, section 3.2.3).
 * cvr_probe_row_read: for each of the n_ids int32 ids (device), reads the
 *   whole row of row_bytes (64, 128 or 256) of the device table at table
 *   (16-byte aligned, n_rows rows), one 16-byte load per lane and eight rows
 *   in flight per lane group -- the access pattern of the embedding gather
 *   over HBM-resident rows (CTR article, section 二).  An id outside
 *   [0, n_rows) reads row 0. */
cvr_status cvr_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t nontemporal,
                                 void* hip_stream);
cvr_status cvr_probe_row_read(const void* table, int64_t n_rows, int32_t row_bytes, const int32_t* ids,
                              int64_t n_ids, uint32_t* sink, int32_t blocks, int32_t nontemporal, void* hip_stream);

const char* cvr_last_error(cvr_handle h);
const char* cvr_status_string(cvr_status s);
void cvr_destroy(cvr_handle h);

#ifdef __cplusplus
}
#endif
#endif /* CVR_H */
