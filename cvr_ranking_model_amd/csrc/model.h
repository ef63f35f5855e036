// Internal state of a libcvr model handle and of one call's workspace layout.
#pragma once
#include <hip/hip_runtime.h>

#include <map>
#include <string>
#include <vector>

#include "../../include/cvr.h"

namespace cvr {

enum Stage {
  STAGE_EXPAND = 0,
  STAGE_GATHER,
  STAGE_MLP_GEMM,
  STAGE_DLRM_OUTPUT,
  STAGE_TOKENIZE_GEMM,
  STAGE_SWIGLU,
  STAGE_SEQ_POOL,
  STAGE_QUERY_GEMM,
  STAGE_ATTENTION,
  STAGE_MIXER_GEMM,
  STAGE_PLE_GEMM,
  STAGE_PLE_GATE,
  STAGE_HEAD_GEMM,
  STAGE_HEAD_OUT,
  STAGE_CACHE,
  STAGE_SEQ_CHUNKS,
  STAGE_EPNET,
  kNumStages
};
constexpr int kMaxLaunchesPerCall = 64;

// One packed dense parameter in the weight arena: a Linear weight matrix [rows][cols] in the
// low-precision type, or a bias vector [rows] in fp32.
struct WEntry {
  std::string name;
  int64_t rows, cols;
  bool matrix;
  size_t off;
  // 0: row-major; 1 / 2: the fused token mixer's first / second Linear in MFMA fragment order
  int pack = 0;
};

// A run of consecutive same-side features in the model input.
struct InputSeg {
  bool item;     // true: item-side matrix; false: request-side matrix read through cand_req
  int k_end;     // end column of the run in the model input
  int col0;      // first column of the run in its side's matrix
};

// Byte offsets of every buffer inside one call's workspace.
struct WsPlan {
  size_t flag = 0, cand_req = 0, x_req = 0, x_item = 0, logits = 0, pooled = 0, pooled_bytes = 0;
  size_t expand_err = 0;      // [expand_blocks] int32: the expand launch's per-block check results
  int64_t expand_blocks = 0;
  size_t h[2] = {0, 0};
  size_t opart = 0;  // DLRM: output-layer partials of a fused last hidden layer
  size_t u_req = 0;  // DLRM with the user block once per request: [R][width 0] fp32
  size_t tok[2] = {0, 0}, hseq = 0, chunk_off = 0, chunk_desc = 0, pool_part = 0, seq_pool = 0, query = 0,
         mixhid = 0, experts = 0, gates = 0, task_in = 0, head_hid = 0, tok_req = 0;
  size_t ep_h = 0, ep_g = 0, x_ep = 0;  // CVR with EPNet: gate hidden, gate pre-activations, scaled input
  // CVR: the first layer's query Linear inputs as bf16 -- the tokenizer's N tokens [n][N][d] and
  // the pools [S][R][d] -- written beside their fp32 forms by the stages that produce them
  size_t xq = 0, pool_bf = 0;
  size_t total = 0;
};

// Graph replay per batch bucket.  A bucket is the batch's four sizes rounded up (bucket_sizes);
// one graph per (bucket, workspace, stream, debug setting) scores the bucket's staging arrays.
struct GraphKey {
  int32_t R = 0, n = 0;
  int64_t ids = 0, P = 0;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t stream = nullptr;
  int debug = 0;
  bool operator==(const GraphKey& o) const {
    return R == o.R && n == o.n && ids == o.ids && P == o.P && ws == o.ws && ws_bytes == o.ws_bytes &&
           stream == o.stream && debug == o.debug;
  }
};
struct GraphEntry {
  GraphKey key;
  hipGraph_t graph = nullptr;
  // two instances of the graph, launched in turn: a replay then never waits for the previous
  // replay of the same instance
  hipGraphExec_t exec[2] = {nullptr, nullptr};
  int next = 0;
  uint64_t used = 0;  // call counter of the last use (least recently used goes first)
  // buffer choices the captured launches made, restored on every replay for cvr_debug_export
  int last_tok = 0, last_attn_tok = 0, last_hidden_buf = 0, last_tok_bf16 = 0;
};
struct GraphCache {
  static constexpr int kMaxGraphs = 8;
  std::vector<GraphEntry> entries;
  uint64_t calls = 0;
  int64_t captures = 0;
  void reset();  // releases every graph
};

// Workspace of a graph-replayed call: the scoring plan at the bucket's sizes, then the bucket's
// staging arrays, score buffer and header.
struct GraphPlan {
  WsPlan plan;
  size_t co = 0, bo = 0, ids = 0, so = 0, scores = 0, hdr = 0, total = 0;
};

struct Timing {
  bool armed = false;
  int max_calls = 0;
  int calls = 0;
  int launch_in_call = 0;
  uint32_t mask = 0;            // stages that carry events (bit per stage); 0 = every stage
  std::vector<hipEvent_t> ev;   // [call][launch][begin,end]
  std::vector<int> stage;       // [call][launch], -1 = unused
  void reset();
};

}  // namespace cvr

struct cvr_model {
  cvr_spec spec{};
  std::vector<cvr_feature> feats;
  std::vector<int32_t> hidden, seq_tables;
  std::vector<int32_t> task_mask;  // CVR: bit e of task_mask[k] set if task k's gate mixes expert e
  std::vector<cvr_table> tables;
  // derived layout
  std::vector<int> fcol;
  int D_req = 0, D_item = 0, ld_req = 0, ld_item = 0, e_dim = 0;
  std::vector<cvr::InputSeg> segs;
  // CVR: the tokenizer split into its request-side and item-side columns (both present and every
  // run a multiple of 32 wide), so requests with many candidates tokenize their own columns once
  bool tok_split = false;
  // CVR with EPNet: runs of context-side (scenario) features in the request-side matrix, their
  // total width
  std::vector<cvr::InputSeg> dom_segs;
  int D_dom = 0;
  // DLRM: the first Linear split into its request-side and item-side columns (both present and
  // every run a multiple of 32 wide), so the request-side product can run once per request
  bool dlrm_split = false;
  // weights
  std::vector<cvr::WEntry> w;
  std::map<std::string, int> widx;
  size_t arena_bytes = 0;
  char* arena = nullptr;
  const void* wptr(const std::string& name) const { return arena + w[widx.at(name)].off; }
  // state
  int debug = 0;
  int64_t pass_rows = -1;  // DLRM candidates per MLP pass: -1 derived from the layer width, 0 one pass
  int opt_tok_share = -1;  // CVR_OPT_TOK_SHARE: -1 auto, 0 off, 1 on
  int opt_attn_mq = -1;    // CVR_OPT_ATTN_MQ: -1 auto, 0 per candidate, 1 MFMA per request
  int opt_user_block = -1; // CVR_OPT_DLRM_USER_BLOCK: -1 auto (off), 0 off, 1 on
  int opt_heads_fused = -1; // CVR_OPT_HEADS_FUSED: -1 auto (fused when the widths allow), 0 off, 1 on
  int opt_state_stream = -1; // CVR_OPT_STATE_STREAM: -1 auto (seq_states_stream), 0 off, 1 on
  std::string err;
  char* last_ws = nullptr;
  cvr::WsPlan last_plan;
  int64_t last_R = 0, last_n = 0, last_P = 0;
  int last_debug = 0, last_tok = 0, last_attn_tok = 0, last_hidden_buf = 0;
  int last_tok_bf16 = 0;  // the last layer's token matrix was written as bf16 (debug off)
  // while a bucket graph is captured: where its sequence encoder finds the caller's seq_ids
  const int32_t* const* capture_seq_ids_ref = nullptr;
  cvr::Timing timing;
  cvr::GraphCache graph;
  // HBM hot-row caches attached to host-resident tables (cvr_cache_attach)
  struct Cache {
    int32_t table;
    int64_t sets;
    int32_t ways;
    char* state;             // caller-owned device memory, laid out by cache_layout
    const float* host_dev;   // device-side address of the host table
  };
  std::vector<Cache> caches;
};

namespace cvr {
WsPlan plan_workspace(const cvr_model* m, int64_t R, int64_t n, int64_t P);
// The bucket of a batch: each size rounded up to the next m * 2^k with 8 <= m <= 16 (sizes
// below 16 exact), one spare request and one spare candidate included.
void bucket_sizes(const cvr_model* m, int64_t R, int64_t n, int64_t ids, int64_t P, int64_t& Rb, int64_t& nb,
                  int64_t& idsb, int64_t& Pb);
GraphPlan plan_graph(const cvr_model* m, int64_t Rb, int64_t nb, int64_t idsb, int64_t Pb);
// Records msg as the handle's (and the thread's) last error and returns s.
cvr_status fail(cvr_model* m, cvr_status s, const std::string& msg);
// cvr_score's work: checks, then the launches into the given workspace.
cvr_status score_call(cvr_handle h, const cvr_batch* b, void* workspace, size_t ws_bytes, float* out_scores,
                      void* hip_stream);
// Candidates per DLRM MLP pass for a batch of n (all of them in debug mode).
int64_t dlrm_pass_rows(const cvr_model* m, int64_t n);

// Times each launch function of one scoring call with a pair of HIP events when timing is armed:
// the events ride on the dispatches themselves (see launch_k); a bracket that launched nothing
// records both events back to back.
struct Launcher {
  cvr_model* m;
  hipStream_t s;
  int slot_base = -1;
  int li = 0;
  Launcher(cvr_model* mm, hipStream_t ss, bool timed = true) : m(mm), s(ss) {
    Timing& t = m->timing;
    if (timed && t.armed && t.calls < t.max_calls) {
      slot_base = t.calls * kMaxLaunchesPerCall;
      t.calls++;
    }
  }
  template <typename F>
  hipError_t operator()(int stage, F&& fn) {
    const uint32_t mask = m->timing.mask;
    const bool rec = slot_base >= 0 && li < kMaxLaunchesPerCall && (mask == 0 || ((mask >> stage) & 1u));
    const size_t slot = (size_t)slot_base + li;
    LaunchTiming& lt = launch_timing();
    if (rec) {
      lt.begin = m->timing.ev[2 * slot];
      lt.end = m->timing.ev[2 * slot + 1];
      lt.launched = 0;
    }
    hipError_t e = fn();
    if (rec) {
      if (lt.launched == 0) {
        (void)hipEventRecord(lt.begin, s);
        (void)hipEventRecord(lt.end, s);
      }
      lt = LaunchTiming{};
      m->timing.stage[slot] = stage;
    }
    li++;
    return e;
  }
};
}  // namespace cvr

hipError_t run_hyformer(cvr_model* m, const cvr_batch* b, char* ws, const cvr::WsPlan& w, float* out,
                        cvr::Launcher& L, hipStream_t s);
