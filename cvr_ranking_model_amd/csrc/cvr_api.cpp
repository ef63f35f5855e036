// Host side of the libcvr C ABI: spec validation, weight packing, workspace planning and the
// per-batch launch sequence.  All device work goes to the caller's stream; no device memory is
// allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/cvr.h"
#include "kernels.h"
#include "model.h"

using namespace cvr;

static thread_local std::string g_last_error;

cvr_status cvr::fail(cvr_model* m, cvr_status s, const std::string& msg) {
  if (m) m->err = msg;
  g_last_error = msg;
  return s;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ------------------------------------------------------------------ spec checks

static bool supported_dim(int d) { return d == 4 || d == 8 || d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

static cvr_status check_spec(const cvr_spec* s, const cvr_table* tables, int32_t n_tables, std::string& why) {
  if (!s) { why = "spec is null"; return CVR_ERR_ARG; }
  if (!tables || n_tables <= 0) { why = "no tables"; return CVR_ERR_ARG; }
  if (s->model != CVR_MODEL_DLRM && s->model != CVR_MODEL_HYFORMER) { why = "unknown model"; return CVR_ERR_SPEC; }
  if (s->lowp != CVR_LOWP_FP16 && s->lowp != CVR_LOWP_BF16) { why = "unknown lowp type"; return CVR_ERR_SPEC; }
  if (!(s->clamp > 0.f) || !std::isfinite(s->clamp)) { why = "clamp bound must be positive"; return CVR_ERR_SPEC; }
  if (s->n_features <= 0 || !s->features) { why = "no features"; return CVR_ERR_SPEC; }
  if (s->n_features > kMaxGatherFeatures) { why = "too many features (max 32)"; return CVR_ERR_UNSUPPORTED; }
  for (int i = 0; i < n_tables; ++i) {
    if (tables[i].rows <= 0 || tables[i].rows > INT32_MAX) { why = "table rows must be in [1, 2^31)"; return CVR_ERR_SPEC; }
    if (!supported_dim(tables[i].dim)) { why = "table dim must be one of 4, 8, 16, 32, 64, 128, 256"; return CVR_ERR_UNSUPPORTED; }
  }
  for (int f = 0; f < s->n_features; ++f) {
    const cvr_feature& F = s->features[f];
    if (F.table < 0 || F.table >= n_tables) { why = "feature table index out of range"; return CVR_ERR_SPEC; }
    if (F.side != CVR_SIDE_USER && F.side != CVR_SIDE_ITEM && F.side != CVR_SIDE_CONTEXT) { why = "bad feature side"; return CVR_ERR_SPEC; }
  }
  if (s->model == CVR_MODEL_DLRM) {
    if (s->lowp != CVR_LOWP_FP16 && s->lowp != CVR_LOWP_BF16) { why = "bad lowp"; return CVR_ERR_SPEC; }
    if (s->n_hidden < 0 || (s->n_hidden > 0 && !s->hidden)) { why = "bad hidden layer list"; return CVR_ERR_SPEC; }
    for (int i = 0; i < s->n_hidden; ++i)
      if (s->hidden[i] <= 0 || s->hidden[i] % 32) { why = "hidden widths must be positive multiples of 32"; return CVR_ERR_UNSUPPORTED; }
  } else {
    // the sequence, attention and token-mixer kernels compute in bf16 (CVR article section 3.4.3)
    if (s->lowp != CVR_LOWP_BF16) { why = "the CVR model runs in bf16 only"; return CVR_ERR_UNSUPPORTED; }
    if (s->d != 128) { why = "token width d must be 128"; return CVR_ERR_UNSUPPORTED; }
    if (s->n_tokens <= 0 || s->n_layers <= 0 || s->n_seq <= 0 || s->n_seq > 4) { why = "bad token/layer/sequence counts"; return CVR_ERR_SPEC; }
    if (s->n_seq_cols <= 0 || !s->seq_tables || s->n_seq_cols > 8) { why = "bad sequence columns"; return CVR_ERR_SPEC; }
    int sd = 0;
    for (int c = 0; c < s->n_seq_cols; ++c) {
      if (s->seq_tables[c] < 0 || s->seq_tables[c] >= n_tables) { why = "sequence table index out of range"; return CVR_ERR_SPEC; }
      sd += tables[s->seq_tables[c]].dim;
    }
    if (sd != s->d) { why = "sequence column dims must sum to d"; return CVR_ERR_SPEC; }
    const int T = s->n_tokens + s->n_seq;
    if (s->mixer_heads <= 0 || s->d % s->mixer_heads || s->d / s->mixer_heads != 8) { why = "mixer heads must split d into chunks of 8"; return CVR_ERR_UNSUPPORTED; }
    if ((T * (s->d / s->mixer_heads)) % 32) { why = "mixed-token width must be a multiple of 32"; return CVR_ERR_UNSUPPORTED; }
    if (s->swiglu_hidden != 256) { why = "SwiGLU hidden width must be 256"; return CVR_ERR_UNSUPPORTED; }
    if (s->mixer_hidden <= 0 || s->mixer_hidden % 32 || s->expert_dim <= 0 || s->expert_dim % 32 ||
        s->head_hidden <= 0 || s->head_hidden % 32) { why = "mixer/expert/head widths must be multiples of 32"; return CVR_ERR_UNSUPPORTED; }
    if (s->n_experts <= 0 || s->n_experts > 8 || s->n_tasks <= 0 || s->n_tasks > 8) { why = "bad expert/task counts"; return CVR_ERR_SPEC; }
    if (s->expert_dim % 64) { why = "expert width must be a multiple of 64"; return CVR_ERR_UNSUPPORTED; }
    if (s->task_experts) {
      for (int k = 0; k < s->n_tasks; ++k) {
        int cnt = 0;
        for (int e = 0; e < s->n_experts; ++e) {
          const int32_t v = s->task_experts[k * s->n_experts + e];
          if (v != 0 && v != 1) { why = "task_experts entries must be 0 or 1"; return CVR_ERR_SPEC; }
          cnt += v;
        }
        if (cnt == 0) { why = "every task must mix at least one expert"; return CVR_ERR_SPEC; }
      }
    }
    if (!(s->tau > 0.f) || !std::isfinite(s->tau)) { why = "tau must be positive"; return CVR_ERR_SPEC; }
    if (s->epnet_hidden < 0) { why = "epnet_hidden must be 0 (off) or positive"; return CVR_ERR_SPEC; }
    if (s->epnet_hidden > 0) {
      if (s->epnet_hidden % 32) { why = "epnet_hidden must be a multiple of 32"; return CVR_ERR_UNSUPPORTED; }
      bool ctx = false;
      for (int f = 0; f < s->n_features; ++f) ctx |= s->features[f].side == CVR_SIDE_CONTEXT;
      if (!ctx) { why = "EPNet needs at least one context-side (scenario) feature"; return CVR_ERR_SPEC; }
    }
  }
  return CVR_OK;
}

// ------------------------------------------------------------------ derived layout

static void derive(cvr_model* m) {
  const cvr_spec& s = m->spec;
  m->fcol.assign(s.n_features, 0);
  m->D_req = m->D_item = 0;
  m->e_dim = 0;
  for (int f = 0; f < s.n_features; ++f) {
    const int dim = m->tables[m->feats[f].table].dim;
    if (m->feats[f].side == CVR_SIDE_ITEM) { m->fcol[f] = m->D_item; m->D_item += dim; }
    else { m->fcol[f] = m->D_req; m->D_req += dim; }
    m->e_dim += dim;
  }
  m->ld_req = (m->D_req + 7) / 8 * 8;
  m->ld_item = (m->D_item + 7) / 8 * 8;
  // K-segments of the model input, merging neighbouring features of the same side.
  m->segs.clear();
  int k = 0;
  for (int f = 0; f < s.n_features; ++f) {
    const int dim = m->tables[m->feats[f].table].dim;
    const bool item = m->feats[f].side == CVR_SIDE_ITEM;
    if (!m->segs.empty() && m->segs.back().item == item) m->segs.back().k_end += dim;
    else m->segs.push_back({item, k + dim, m->fcol[f]});
    k += dim;
  }
  // EPNet's scenario columns: runs of consecutive context-side features in the request-side matrix
  m->dom_segs.clear();
  m->D_dom = 0;
  if (s.model == CVR_MODEL_HYFORMER && s.epnet_hidden > 0) {
    int run_k0 = 0;  // first gate-input column of the current run
    for (int f = 0; f < s.n_features; ++f) {
      if (m->feats[f].side != CVR_SIDE_CONTEXT) continue;
      const int dim = m->tables[m->feats[f].table].dim;
      const bool extends = !m->dom_segs.empty() && m->dom_segs.back().col0 + (m->D_dom - run_k0) == m->fcol[f];
      if (extends) {
        m->dom_segs.back().k_end += dim;
      } else {
        run_k0 = m->D_dom;
        m->dom_segs.push_back({false, m->D_dom + dim, m->fcol[f]});
      }
      m->D_dom += dim;
    }
  }
  // the tokenizer's request-side block once per request: not with EPNet, whose scale is per candidate
  m->tok_split = s.model == CVR_MODEL_HYFORMER && m->D_req > 0 && m->D_item > 0 && s.epnet_hidden == 0;
  m->dlrm_split = s.model == CVR_MODEL_DLRM && m->D_req > 0 && m->D_item > 0 && s.n_hidden > 0;
  int kb = 0;
  for (const InputSeg& sg : m->segs) {
    if ((sg.k_end - kb) % 32) m->tok_split = m->dlrm_split = false;
    kb = sg.k_end;
  }
}

// Weight arena plan.  Entries listed together are placed back to back so that grouped GEMMs
// can step through them with one stride.
static void plan_weights(cvr_model* m) {
  const cvr_spec& s = m->spec;
  m->w.clear();
  m->widx.clear();
  size_t off = 0;
  auto add = [&](const std::string& name, int64_t rows, int64_t cols, bool matrix) {
    WEntry e{name, rows, cols, matrix, off};
    off = align256(off + (size_t)rows * cols * (matrix ? 2 : 4));
    m->widx[name] = (int)m->w.size();
    m->w.push_back(e);
  };
  if (s.model == CVR_MODEL_DLRM) {
    int in = m->e_dim;
    for (int i = 0; i <= s.n_hidden; ++i) {
      const int out = i < s.n_hidden ? m->hidden[i] : 1;
      add("mlp." + std::to_string(i) + ".weight", out, in, true);
      add("mlp." + std::to_string(i) + ".bias", out, 1, false);
      if (i == 0 && m->dlrm_split) {
        // the first Linear's request-side and item-side columns as matrices of their own
        add("_mlp0.req.weight", out, m->D_req, true);
        add("_mlp0.item.weight", out, m->D_item, true);
      }
      in = out;
    }
  } else {
    const int d = s.d, N = s.n_tokens, S = s.n_seq, T = N + S, hs = s.swiglu_hidden;
    const int mw = T * d / s.mixer_heads;
    if (s.epnet_hidden > 0) {
      add("epnet.fc1.weight", s.epnet_hidden, (int64_t)m->D_dom + m->e_dim, true);
      add("epnet.fc1.bias", s.epnet_hidden, 1, false);
      add("epnet.fc2.weight", m->e_dim, s.epnet_hidden, true);
      add("epnet.fc2.bias", m->e_dim, 1, false);
    }
    add("tok.weight", (int64_t)N * d, m->e_dim, true);
    add("tok.bias", (int64_t)N * d, 1, false);
    if (m->tok_split) {
      // the tokenizer's request-side and item-side columns as matrices of their own
      add("_tok.req.weight", (int64_t)N * d, m->D_req, true);
      add("_tok.item.weight", (int64_t)N * d, m->D_item, true);
    }
    for (int q = 0; q < S; ++q) {
      // gate and up back to back: one [2*hs][d] matrix per sequence
      add("seq." + std::to_string(q) + ".gate.weight", hs, d, true);
      add("seq." + std::to_string(q) + ".up.weight", hs, d, true);
      add("seq." + std::to_string(q) + ".gate.bias", hs, 1, false);
      add("seq." + std::to_string(q) + ".up.bias", hs, 1, false);
      add("seq." + std::to_string(q) + ".down.weight", d, hs, true);
      add("seq." + std::to_string(q) + ".down.bias", d, 1, false);
    }
    for (int l = 0; l < s.n_layers; ++l) {
      const std::string L = "layer." + std::to_string(l);
      for (int q = 0; q < S; ++q) add(L + ".query." + std::to_string(q) + ".weight", d, (int64_t)(N + 1) * d, true);
      for (int q = 0; q < S; ++q) add(L + ".query." + std::to_string(q) + ".bias", d, 1, false);
      for (int h = 0; h < s.mixer_heads; ++h) add(L + ".mix." + std::to_string(h) + ".fc1.weight", s.mixer_hidden, mw, true);
      for (int h = 0; h < s.mixer_heads; ++h) add(L + ".mix." + std::to_string(h) + ".fc1.bias", s.mixer_hidden, 1, false);
      for (int h = 0; h < s.mixer_heads; ++h) add(L + ".mix." + std::to_string(h) + ".fc2.weight", mw, s.mixer_hidden, true);
      for (int h = 0; h < s.mixer_heads; ++h) add(L + ".mix." + std::to_string(h) + ".fc2.bias", mw, 1, false);
      if (token_mix_supported(T, d, s.mixer_heads, s.mixer_hidden))
        for (int h = 0; h < s.mixer_heads; ++h) {
          m->w[m->widx.at(L + ".mix." + std::to_string(h) + ".fc1.weight")].pack = 1;
          m->w[m->widx.at(L + ".mix." + std::to_string(h) + ".fc2.weight")].pack = 2;
        }
    }
    const int zd = T * d;
    // Expert rows, then every task's gate rows, back to back: one GEMM computes the experts and
    // the gate logits.  Its bias vector is the internal entry "_ple.bias" (expert biases, then
    // gate biases), assembled from the given biases at create time.
    int gates = 0;
    for (int e = 0; e < s.n_experts; ++e) add("ple.expert." + std::to_string(e) + ".weight", s.expert_dim, zd, true);
    for (int k = 0; k < s.n_tasks; ++k) {
      add("ple.gate." + std::to_string(k) + ".weight", __builtin_popcount(m->task_mask[k]), zd, true);
      gates += __builtin_popcount(m->task_mask[k]);
    }
    for (int e = 0; e < s.n_experts; ++e) add("ple.expert." + std::to_string(e) + ".bias", s.expert_dim, 1, false);
    for (int k = 0; k < s.n_tasks; ++k) add("ple.gate." + std::to_string(k) + ".bias", __builtin_popcount(m->task_mask[k]), 1, false);
    add("_ple.bias", (int64_t)s.n_experts * s.expert_dim + gates, 1, false);
    for (int k = 0; k < s.n_tasks; ++k) add("head." + std::to_string(k) + ".fc1.weight", s.head_hidden, s.expert_dim, true);
    for (int k = 0; k < s.n_tasks; ++k) add("head." + std::to_string(k) + ".fc1.bias", s.head_hidden, 1, false);
    for (int k = 0; k < s.n_tasks; ++k) add("head." + std::to_string(k) + ".fc2.weight", 1, s.head_hidden, true);
    for (int k = 0; k < s.n_tasks; ++k) add("head." + std::to_string(k) + ".fc2.bias", 1, 1, false);
  }
  m->arena_bytes = align256(off);
}

static cvr_model* new_model(const cvr_spec* spec, const cvr_table* tables, int32_t n_tables) {
  cvr_model* m = new cvr_model();
  m->spec = *spec;
  m->feats.assign(spec->features, spec->features + spec->n_features);
  m->spec.features = m->feats.data();
  if (spec->model == CVR_MODEL_DLRM && spec->n_hidden > 0) m->hidden.assign(spec->hidden, spec->hidden + spec->n_hidden);
  m->spec.hidden = m->hidden.data();
  if (spec->model == CVR_MODEL_HYFORMER) m->seq_tables.assign(spec->seq_tables, spec->seq_tables + spec->n_seq_cols);
  m->spec.seq_tables = m->seq_tables.data();
  if (spec->model == CVR_MODEL_HYFORMER) {
    m->task_mask.assign(spec->n_tasks, 0);
    for (int k = 0; k < spec->n_tasks; ++k)
      for (int e = 0; e < spec->n_experts; ++e)
        if (!spec->task_experts || spec->task_experts[k * spec->n_experts + e]) m->task_mask[k] |= 1 << e;
  }
  m->spec.task_experts = nullptr;  // the caller's array is not kept; task_mask holds it
  m->tables.assign(tables, tables + n_tables);
  derive(m);
  plan_weights(m);
  return m;
}

static cvr_status check_segments(const cvr_model* m, std::string& why) {
  if (m->segs.size() > (size_t)kMaxASegments) { why = "model input alternates sides too often (max 4 runs)"; return CVR_ERR_UNSUPPORTED; }
  for (const auto& sg : m->segs)
    if (sg.k_end % 32 || sg.col0 % 8) { why = "each run of same-side features must end on a multiple of 32 columns"; return CVR_ERR_UNSUPPORTED; }
  if (m->e_dim % 32) { why = "model input width must be a multiple of 32"; return CVR_ERR_UNSUPPORTED; }
  if (!m->dom_segs.empty()) {
    if (m->dom_segs.size() + m->segs.size() > (size_t)kMaxASegments)
      { why = "EPNet: scenario runs plus input runs exceed 4 segments"; return CVR_ERR_UNSUPPORTED; }
    for (const auto& sg : m->dom_segs)
      if (sg.k_end % 32 || sg.col0 % 8) { why = "EPNet: each run of scenario features must be a multiple of 32 wide"; return CVR_ERR_UNSUPPORTED; }
  }
  return CVR_OK;
}

extern "C" cvr_status cvr_weight_arena_bytes(const cvr_spec* spec, const cvr_table* tables, int32_t n_tables,
                                             size_t* bytes) {
  std::string why;
  if (!bytes) return fail(nullptr, CVR_ERR_ARG, "bytes is null");
  cvr_status st = check_spec(spec, tables, n_tables, why);
  if (st != CVR_OK) return fail(nullptr, st, why);
  cvr_model* m = new_model(spec, tables, n_tables);
  *bytes = m->arena_bytes;
  delete m;
  return CVR_OK;
}

extern "C" cvr_status cvr_create(const cvr_spec* spec, const cvr_table* tables, int32_t n_tables,
                                 const cvr_weight* weights, int32_t n_weights, void* weight_arena,
                                 size_t arena_bytes, void* hip_stream, cvr_handle* out) {
  if (!out) return fail(nullptr, CVR_ERR_ARG, "out is null");
  *out = nullptr;
  std::string why;
  cvr_status st = check_spec(spec, tables, n_tables, why);
  if (st != CVR_OK) return fail(nullptr, st, why);
  for (int i = 0; i < n_tables; ++i)
    if (!tables[i].data || ((uintptr_t)tables[i].data & 15)) return fail(nullptr, CVR_ERR_ARG, "table data must be non-null and 16-byte aligned");
  cvr_model* m = new_model(spec, tables, n_tables);
  // Kernels read tables at device addresses: device memory is used as is, pinned host memory
  // (a table kept in host DRAM) through its device-side address; memory HIP does not know
  // (pageable host memory) cannot be read by a kernel and is refused.
  for (int i = 0; i < n_tables; ++i) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, tables[i].data) != hipSuccess) {
      (void)hipGetLastError();
      delete m;
      return fail(nullptr, CVR_ERR_ARG, "table " + std::to_string(i) + " is neither device memory nor pinned host memory");
    }
    if (attr.type == hipMemoryTypeHost) {
      void* p = nullptr;
      if (hipHostGetDevicePointer(&p, (void*)tables[i].data, 0) != hipSuccess || !p) {
        (void)hipGetLastError();
        delete m;
        return fail(nullptr, CVR_ERR_ARG, "table " + std::to_string(i) + ": host memory without a device address");
      }
      m->tables[i].data = (const float*)p;
    }
  }
  st = check_segments(m, why);
  if (st != CVR_OK) { delete m; return fail(nullptr, st, why); }
  if (!weight_arena || ((uintptr_t)weight_arena & 255)) { delete m; return fail(nullptr, CVR_ERR_ARG, "weight arena must be non-null and 256-byte aligned"); }
  if (arena_bytes < m->arena_bytes) { delete m; return fail(nullptr, CVR_ERR_WORKSPACE, "weight arena too small"); }
  if (!weights || n_weights <= 0) { delete m; return fail(nullptr, CVR_ERR_SPEC, "no weights given"); }
  m->arena = (char*)weight_arena;
  hipStream_t s = (hipStream_t)hip_stream;
  std::vector<int> seen(m->w.size(), 0);
  for (int i = 0; i < n_weights; ++i) {
    if (!weights[i].name) { delete m; return fail(nullptr, CVR_ERR_ARG, "weight without a name"); }
    auto it = m->widx.find(weights[i].name);
    if (it == m->widx.end()) { std::string n = weights[i].name; delete m; return fail(nullptr, CVR_ERR_SPEC, "unexpected weight " + n); }
    const WEntry& e = m->w[it->second];
    if (weights[i].numel != e.rows * e.cols) {
      std::string n = weights[i].name; delete m;
      return fail(nullptr, CVR_ERR_SPEC, "weight " + n + " has " + std::to_string(weights[i].numel) + " elements, expected " + std::to_string(e.rows * e.cols));
    }
    if (!weights[i].data) { delete m; return fail(nullptr, CVR_ERR_ARG, "weight data is null"); }
    if (seen[it->second]++) { std::string n = weights[i].name; delete m; return fail(nullptr, CVR_ERR_SPEC, "weight given twice: " + n); }
    hipError_t he;
    if (e.pack) he = launch_mix_pack(weights[i].data, m->arena + e.off, e.pack, s);
    else if (e.matrix) he = launch_convert(weights[i].data, m->arena + e.off, e.rows * e.cols, m->spec.lowp, s);
    else he = hipMemcpyAsync(m->arena + e.off, weights[i].data, (size_t)e.rows * 4, hipMemcpyDeviceToDevice, s);
    if (he != hipSuccess) { delete m; return fail(nullptr, CVR_ERR_HIP, std::string("packing weights: ") + hipGetErrorString(he)); }
  }
  for (size_t i = 0; i < seen.size(); ++i)
    if (!seen[i] && m->w[i].name[0] != '_') { std::string n = m->w[i].name; delete m; return fail(nullptr, CVR_ERR_SPEC, "missing weight " + n); }
  // column runs of a packed input-side weight (the tokenizer's, or the first MLP layer's) into its
  // request-side and item-side matrices
  const char* split_src = m->tok_split ? "tok.weight" : (m->dlrm_split ? "mlp.0.weight" : nullptr);
  if (split_src) {
    const std::string pre = m->tok_split ? "_tok" : "_mlp0";
    const WEntry& wt = m->w[m->widx.at(split_src)];
    const WEntry& wr = m->w[m->widx.at(pre + ".req.weight")];
    const WEntry& wi = m->w[m->widx.at(pre + ".item.weight")];
    int kb = 0, creq = 0, citem = 0;
    for (const InputSeg& sg : m->segs) {
      const int width = sg.k_end - kb;
      const WEntry& dst = sg.item ? wi : wr;
      int& c = sg.item ? citem : creq;
      hipError_t he = hipMemcpy2DAsync(m->arena + dst.off + (size_t)c * 2, (size_t)dst.cols * 2,
                                       m->arena + wt.off + (size_t)kb * 2, (size_t)wt.cols * 2, (size_t)width * 2,
                                       (size_t)wt.rows, hipMemcpyDeviceToDevice, s);
      if (he != hipSuccess) { delete m; return fail(nullptr, CVR_ERR_HIP, std::string("splitting input weight: ") + hipGetErrorString(he)); }
      c += width;
      kb = sg.k_end;
    }
  }
  if (m->spec.model == CVR_MODEL_HYFORMER) {
    // the expert GEMM's bias vector: expert biases, then the gate biases task by task
    char* dst = m->arena + m->w[m->widx.at("_ple.bias")].off;
    std::vector<std::string> parts;
    for (int e = 0; e < m->spec.n_experts; ++e) parts.push_back("ple.expert." + std::to_string(e) + ".bias");
    for (int k = 0; k < m->spec.n_tasks; ++k) parts.push_back("ple.gate." + std::to_string(k) + ".bias");
    for (const std::string& name : parts) {
      const WEntry& e = m->w[m->widx.at(name)];
      hipError_t he = hipMemcpyAsync(dst, m->arena + e.off, (size_t)e.rows * 4, hipMemcpyDeviceToDevice, s);
      if (he != hipSuccess) { delete m; return fail(nullptr, CVR_ERR_HIP, std::string("packing biases: ") + hipGetErrorString(he)); }
      dst += (size_t)e.rows * 4;
    }
  }
  hipError_t he = hipStreamSynchronize(s);
  if (he != hipSuccess) { delete m; return fail(nullptr, CVR_ERR_HIP, std::string("create sync: ") + hipGetErrorString(he)); }
  *out = m;
  return CVR_OK;
}

// ------------------------------------------------------------------ workspace

// The DLRM MLP runs all its layers over one slice of candidates before the next slice, so
// its two activation buffers hold one slice rather than the whole batch.  A slice is sized so
// that one buffer takes at most 128 MB (65536 candidates at width 1024, fp16): at 128k
// candidates the whole-batch buffers (2 x 256 MB) would stream through the 256 MB
// last-level cache on every layer, while two slices keep their buffers there.  Each slice
// costs one more launch per layer, so slices are no smaller than that.  The result does not
// depend on the split: each candidate's row is computed by the same arithmetic in any slice.
// The slice never grows with n, so a workspace sized for a batch serves every smaller one.
int64_t cvr::dlrm_pass_rows(const cvr_model* m, int64_t n) {
  if (m->debug || m->pass_rows == 0) return n;
  int64_t rows = m->pass_rows;
  if (rows < 0) {
    int maxw = 1;
    for (int i = 0; i < m->spec.n_hidden; ++i) maxw = std::max(maxw, m->hidden[i]);
    rows = std::max<int64_t>(256, ((int64_t)128 << 20) / ((int64_t)maxw * 2) / 256 * 256);
  }
  return std::min(n, rows);
}

WsPlan cvr::plan_workspace(const cvr_model* m, int64_t R, int64_t n, int64_t P) {
  const cvr_spec& s = m->spec;
  WsPlan w;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t lp = 2;
  w.flag = take(256);
  {
    int64_t bags = 0;
    for (int f = 0; f < s.n_features; ++f) bags += m->feats[f].side == CVR_SIDE_ITEM ? n : R;
    w.expand_blocks = expand_blocks(n, bags, R, s.model == CVR_MODEL_HYFORMER ? s.n_seq : 0);
    w.expand_err = take((size_t)w.expand_blocks * 4);
  }
  w.cand_req = take((size_t)n * 4);
  w.x_req = take((size_t)R * m->ld_req * lp);
  w.x_item = take((size_t)n * m->ld_item * lp);
  const int ntasks = s.model == CVR_MODEL_DLRM ? 1 : s.n_tasks;
  w.logits = take((size_t)n * ntasks * 4);
  size_t pooled = 0;
  for (int f = 0; f < s.n_features; ++f)
    pooled += (size_t)(m->feats[f].side == CVR_SIDE_ITEM ? n : R) * m->tables[m->feats[f].table].dim * 4;
  w.pooled = m->debug ? take(pooled) : 0;
  w.pooled_bytes = m->debug ? pooled : 0;
  if (s.model == CVR_MODEL_DLRM) {
    int maxw = 1;
    for (int i = 0; i < s.n_hidden; ++i) maxw = std::max(maxw, m->hidden[i]);
    const int64_t hr = dlrm_pass_rows(m, n);
    w.h[0] = take((size_t)hr * maxw * lp);
    w.h[1] = take((size_t)hr * maxw * lp);
    const int wl = s.n_hidden > 0 ? m->hidden[s.n_hidden - 1] : 0;
    w.opart = take((size_t)((wl + kOutGroup - 1) / kOutGroup) * hr * 4);
    if (m->dlrm_split) w.u_req = take((size_t)R * m->hidden[0] * 4);
  } else {
    const int64_t d = s.d, S = s.n_seq, T = s.n_tokens + s.n_seq;
    w.tok[0] = take((size_t)n * T * d * 4);
    w.tok[1] = take((size_t)n * T * d * 4);
    w.tok_req = take((size_t)R * s.n_tokens * d * 4);
    w.hseq = take((size_t)P * d * lp);
    w.chunk_off = take((size_t)(S * R + 1) * 4);
    w.pool_part = take((size_t)(P / kSeqChunk + S * R + 1) * d * 4);
    w.chunk_desc = take((size_t)(P / kSeqChunk + S * R + 1) * 8);
    w.seq_pool = take((size_t)S * R * d * 4);
    w.pool_bf = take((size_t)S * R * d * lp);
    w.xq = take((size_t)n * s.n_tokens * d * lp);
    w.query = take((size_t)S * n * d * 4);
    w.mixhid = take((size_t)s.mixer_heads * n * s.mixer_hidden * lp);
    w.experts = take((size_t)n * ((s.n_experts * s.expert_dim + s.n_tasks * s.n_experts + 31) / 32 * 32) * 4);
    w.gates = take((size_t)n * s.n_tasks * s.n_experts * 4);
    w.task_in = take((size_t)s.n_tasks * n * s.expert_dim * lp);
    w.head_hid = take((size_t)s.n_tasks * n * s.head_hidden * lp);
    if (s.epnet_hidden > 0) {
      w.ep_h = take((size_t)n * s.epnet_hidden * lp);
      w.ep_g = take((size_t)n * m->e_dim * 4);
      w.x_ep = take((size_t)n * m->e_dim * lp);
    }
  }
  w.total = align256(off);
  return w;
}

extern "C" cvr_status cvr_workspace_bytes(cvr_handle h, int32_t max_requests, int32_t max_candidates, int64_t max_ids,
                                          int64_t max_positions, size_t* bytes) {
  if (!h || !bytes) return fail(h, CVR_ERR_ARG, "null argument");
  if (max_requests < 0 || max_candidates < 0 || max_ids < 0 || max_positions < 0) return fail(h, CVR_ERR_ARG, "negative size");
  *bytes = plan_workspace(h, max_requests, max_candidates, h->spec.model == CVR_MODEL_DLRM ? 0 : max_positions).total;
  return CVR_OK;
}

// ------------------------------------------------------------------ timing
LaunchTiming& cvr::launch_timing() {
  static thread_local LaunchTiming t;
  return t;
}


void Timing::reset() {
  for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  ev.clear();
  stage.clear();
  armed = false;
  calls = 0;
  max_calls = 0;
  launch_in_call = 0;
  mask = 0;
}

extern "C" cvr_status cvr_timing_begin(cvr_handle h, int32_t max_calls, uint32_t stage_mask) {
  if (!h || max_calls <= 0 || max_calls > 100000) return fail(h, CVR_ERR_ARG, "bad timing request");
  if (stage_mask >> kNumStages) return fail(h, CVR_ERR_ARG, "timing mask names an unknown stage");
  h->timing.reset();
  h->timing.mask = stage_mask;
  h->timing.ev.resize((size_t)max_calls * kMaxLaunchesPerCall * 2);
  h->timing.stage.assign((size_t)max_calls * kMaxLaunchesPerCall, -1);
  for (auto& e : h->timing.ev)
    if (hipEventCreate(&e) != hipSuccess) { h->timing.ev.clear(); return fail(h, CVR_ERR_HIP, "hipEventCreate failed"); }
  h->timing.max_calls = max_calls;
  h->timing.armed = true;
  return CVR_OK;
}

extern "C" cvr_status cvr_timing_end(cvr_handle h, double* stage_ms, int32_t* stage_launches, int32_t max_stages,
                                     int32_t* n_stages, int32_t* n_calls) {
  if (!h) return fail(h, CVR_ERR_ARG, "null handle");
  Timing& t = h->timing;
  std::vector<double> ms(kNumStages, 0.0);
  std::vector<int> cnt(kNumStages, 0);
  for (int c = 0; c < t.calls; ++c)
    for (int l = 0; l < kMaxLaunchesPerCall; ++l) {
      const size_t slot = (size_t)c * kMaxLaunchesPerCall + l;
      const int st = t.stage[slot];
      if (st < 0) continue;
      if (hipEventSynchronize(t.ev[2 * slot + 1]) != hipSuccess) return fail(h, CVR_ERR_HIP, "event sync failed");
      float f = 0.f;
      if (hipEventElapsedTime(&f, t.ev[2 * slot], t.ev[2 * slot + 1]) != hipSuccess) return fail(h, CVR_ERR_HIP, "elapsed time failed");
      ms[st] += f;
      cnt[st] += 1;
    }
  for (int i = 0; i < kNumStages && i < max_stages; ++i) {
    if (stage_ms) stage_ms[i] = ms[i];
    if (stage_launches) stage_launches[i] = cnt[i];
  }
  if (n_stages) *n_stages = kNumStages;
  if (n_calls) *n_calls = t.calls;
  t.reset();
  return CVR_OK;
}

extern "C" const char* cvr_stage_name(cvr_handle, int32_t stage) {
  static const char* names[kNumStages] = {"expand", "gather_pool", "mlp_gemm", "dlrm_output", "tokenize_gemm",
                                          "swiglu", "seq_pool", "query_gemm", "attention", "mixer_gemm",
                                          "ple_gemm", "ple_gate", "head_gemm", "head_out", "cache", "seq_chunks",
                                          "epnet"};
  return (stage >= 0 && stage < kNumStages) ? names[stage] : "";
}

// ------------------------------------------------------------------ scoring


static cvr_status check_batch_args(cvr_model* m, const cvr_batch* b, void* ws, float* out) {
  if (!b || !ws || !out) return fail(m, CVR_ERR_ARG, "null batch, workspace or output");
  if ((uintptr_t)ws & 255) return fail(m, CVR_ERR_ARG, "workspace must be 256-byte aligned");
  if (b->n_requests <= 0) return fail(m, CVR_ERR_ARG, "n_requests must be >= 1");
  if (b->n_candidates < 0 || b->n_ids < 0 || b->n_positions < 0) return fail(m, CVR_ERR_ARG, "negative size");
  if (b->n_ids > INT32_MAX || b->n_positions > INT32_MAX) return fail(m, CVR_ERR_ARG, "ids/positions must fit int32");
  if (!b->cand_offsets || !b->bag_offsets || (b->n_ids > 0 && !b->ids)) return fail(m, CVR_ERR_ARG, "null CSR array");
  if (m->spec.model == CVR_MODEL_HYFORMER && (!b->seq_offsets || (b->n_positions > 0 && !b->seq_ids)))
    return fail(m, CVR_ERR_ARG, "CVR model needs seq_offsets and seq_ids");
  // chunk descriptors carry the (sequence, request) segment in 23 bits
  if (m->spec.model == CVR_MODEL_HYFORMER && (int64_t)m->spec.n_seq * b->n_requests >= (1 << 23))
    return fail(m, CVR_ERR_ARG, "n_seq * n_requests must be below 2^23");
  return CVR_OK;
}

static cvr_status check_batch(cvr_model* m, const cvr_batch* b, void* ws, size_t ws_bytes, float* out, WsPlan& plan) {
  cvr_status st = check_batch_args(m, b, ws, out);
  if (st != CVR_OK) return st;
  plan = plan_workspace(m, b->n_requests, b->n_candidates, m->spec.model == CVR_MODEL_DLRM ? 0 : b->n_positions);
  if (ws_bytes < plan.total) return fail(m, CVR_ERR_WORKSPACE, "workspace too small: need " + std::to_string(plan.total) + " bytes");
  return CVR_OK;
}

static GatherCache gather_cache(const cvr_model::Cache& c, int32_t dim) {
  const CacheLayout l = cache_layout(c.sets, c.ways, dim);
  GatherCache g{};
  g.hdr = (CacheHeader*)c.state;
  g.tags = (int32_t*)(c.state + l.tags);
  g.stamps = (int32_t*)(c.state + l.stamps);
  g.first = (int32_t*)(c.state + l.first);
  g.queue = (int32_t*)(c.state + l.queue);
  g.rows = (float*)(c.state + l.rows);
  g.sets = (int32_t)c.sets;
  g.ways = c.ways;
  return g;
}

// Shared front of both models: flag clear, expand, gather-pool into the two input matrices.
// bucket: the batch is a graph bucket's padded staging copy, whose n_ids is a capacity (its last
// bag may end before it).
static hipError_t run_front(cvr_model* m, const cvr_batch* b, char* ws, const WsPlan& w, Launcher& L, hipStream_t s,
                            bool bucket = false) {
  const cvr_spec& sp = m->spec;
  int32_t* flag = (int32_t*)(ws + w.flag);
  int64_t total_bags = 0;
  for (int f = 0; f < sp.n_features; ++f) total_bags += sp.features[f].side == CVR_SIDE_ITEM ? b->n_candidates : b->n_requests;
  ExpandParams ep{};
  ep.cand_offsets = b->cand_offsets;
  ep.R = b->n_requests;
  ep.n = b->n_candidates;
  ep.bag_offsets = b->bag_offsets;
  ep.total_bags = total_bags;
  ep.n_ids = b->n_ids;
  ep.seq_offsets = sp.model == CVR_MODEL_HYFORMER ? b->seq_offsets : nullptr;
  ep.S = sp.model == CVR_MODEL_HYFORMER ? sp.n_seq : 0;
  ep.n_positions = b->n_positions;
  ep.cand_req = (int32_t*)(ws + w.cand_req);
  ep.flag = flag;
  ep.block_err = (int32_t*)(ws + w.expand_err);
  ep.ids_capacity = bucket ? 1 : 0;
  hipError_t e;
  if (sp.model == CVR_MODEL_HYFORMER && seq_plan_in_front(sp.n_seq, b->n_requests)) {
    // the sequence chunk plan reads only the sequence offsets: it runs beside the expansion
    const int64_t max_chunks = b->n_positions / kSeqChunk + (int64_t)sp.n_seq * b->n_requests;
    if (max_chunks > INT32_MAX) return hipErrorInvalidValue;
    PlanParams q{b->seq_offsets, b->n_requests, sp.n_seq, b->n_positions, (int32_t)max_chunks,
                 (int32_t*)(ws + w.chunk_off), (int2*)(ws + w.chunk_desc)};
    e = L(STAGE_EXPAND, [&] { return launch_front(ep, w.expand_blocks, q, s); });
  } else {
    e = L(STAGE_EXPAND, [&] { return launch_expand(ep, w.expand_blocks, s); });
  }
  if (e != hipSuccess) return e;

  GatherParams gp{};
  gp.nf = sp.n_features;
  gp.bag_offsets = b->bag_offsets;
  gp.ids = b->ids;
  gp.n_ids = b->n_ids;
  gp.clamp = sp.clamp;
  gp.lowp = sp.lowp;
  gp.flag = flag;
  CacheHeader* hdrs[kMaxCaches];
  for (size_t c = 0; c < m->caches.size(); ++c) {
    gp.cache[c] = gather_cache(m->caches[c], m->tables[m->caches[c].table].dim);
    hdrs[c] = gp.cache[c].hdr;
  }
  if (!m->caches.empty()) {
    e = L(STAGE_CACHE, [&] { return launch_cache_begin(hdrs, (int)m->caches.size(), s); });
    if (e != hipSuccess) return e;
  }
  int64_t base = 0;
  size_t dbg = w.pooled;
  for (int f = 0; f < sp.n_features; ++f) {
    const cvr_table& t = m->tables[sp.features[f].table];
    const bool item = sp.features[f].side == CVR_SIDE_ITEM;
    GatherFeature& F = gp.f[f];
    F.cache = -1;
    F.table = t.data;
    for (size_t c = 0; c < m->caches.size(); ++c)
      if (m->caches[c].table == sp.features[f].table) {
        F.cache = (int32_t)c;
        F.table = m->caches[c].host_dev;
      }
    F.rows = t.rows;
    F.dim = t.dim;
    F.nbags = item ? b->n_candidates : b->n_requests;
    F.bag_base = base;
    F.out = ws + (item ? w.x_item : w.x_req);
    F.ldo = item ? m->ld_item : m->ld_req;
    F.col = m->fcol[f];
    F.dbg = m->debug ? (float*)(ws + dbg) : nullptr;
    dbg += (size_t)F.nbags * t.dim * 4;
    base += F.nbags;
  }
  e = L(STAGE_GATHER, [&] { return launch_gather_pool(gp, s); });
  if (e != hipSuccess) return e;
  for (size_t c = 0; c < m->caches.size(); ++c) {
    const cvr_model::Cache& mc = m->caches[c];
    e = L(STAGE_CACHE, [&] {
      return launch_cache_admit(gp.cache[c], b->ids, b->n_ids, mc.host_dev, m->tables[mc.table].rows,
                                m->tables[mc.table].dim, b->n_ids, s);
    });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The model input as GEMM K-segments (request-side runs read through cand_req).
// Candidate rows r0.. of the model input: item columns are read in place, request columns
// through the candidate -> request map.
static void input_segments(const cvr_model* m, char* ws, const WsPlan& w, GemmParams& g, int64_t r0 = 0) {
  g.nseg = (int)m->segs.size();
  for (size_t i = 0; i < m->segs.size(); ++i) {
    const InputSeg& sg = m->segs[i];
    ASeg& a = g.seg[i];
    a.ptr = sg.item ? ws + w.x_item + (size_t)r0 * m->ld_item * 2 : ws + w.x_req;
    a.rowmap = sg.item ? nullptr : (const int32_t*)(ws + w.cand_req) + r0;
    a.ld = sg.item ? m->ld_item : m->ld_req;
    a.gstride = 0;
    a.k_end = sg.k_end;
    a.kstride8 = 8;
    a.col0 = sg.col0;
  }
}

static hipError_t run_dlrm(cvr_model* m, const cvr_batch* b, char* ws, const WsPlan& w, float* out, Launcher& L,
                           hipStream_t s) {
  const cvr_spec& sp = m->spec;
  const int64_t n = b->n_candidates;
  const int64_t pr = dlrm_pass_rows(m, n);
  if (sp.n_hidden < 1) return hipErrorInvalidValue;  // zero hidden layers: not supported by the output kernel
  hipError_t e = hipSuccess;
  const int L_ = sp.n_hidden;
  const void* w_out = m->wptr("mlp." + std::to_string(L_) + ".weight");
  const float* b_out = (const float*)m->wptr("mlp." + std::to_string(L_) + ".bias");
  // The user block (CTR article section 四; CVR article section 3.4.5, taken to the first layer):
  // the request-side columns of the first Linear multiplied once per request, U = X_req W_req^T
  // in fp32; every candidate's first layer adds its request's row of U to its item-side product.
  const bool user_block = m->dlrm_split && m->opt_user_block == 1;
  if (user_block) {
    GemmParams g{};
    g.M = b->n_requests;
    g.N = m->hidden[0];
    g.K = m->D_req;
    g.groups = 1;
    int kb = 0, k = 0;
    for (const InputSeg& sg : m->segs) {
      if (!sg.item) {
        k += sg.k_end - kb;
        g.seg[g.nseg++] = ASeg{ws + w.x_req, nullptr, (int64_t)m->ld_req, 0, k, 8, sg.col0, 0};
      }
      kb = sg.k_end;
    }
    g.W = m->wptr("_mlp0.req.weight");
    g.C = ws + w.u_req;
    g.ldc = m->hidden[0];
    g.c_nstride8 = 8;
    g.out_f32 = 1;
    e = L(STAGE_MLP_GEMM, [&] { return launch_gemm(g, sp.lowp, s); });
    if (e != hipSuccess) return e;
  }
  for (int64_t r0 = 0; r0 < n; r0 += pr) {
    const int mc = (int)std::min(pr, n - r0);
    int in = m->e_dim;
    int cur = -1;
    bool fused = false;
    for (int i = 0; i < sp.n_hidden; ++i) {
      const int width = m->hidden[i];
      GemmParams g{};
      g.M = mc;
      g.N = width;
      g.K = in;
      g.groups = 1;
      g.W = m->wptr("mlp." + std::to_string(i) + ".weight");
      if (i == 0 && user_block) {
        // item-side columns only, plus the request's row of U
        g.K = m->D_item;
        int kb = 0, k = 0;
        for (const InputSeg& sg : m->segs) {
          if (sg.item) {
            k += sg.k_end - kb;
            g.seg[g.nseg++] = ASeg{ws + w.x_item + (size_t)r0 * m->ld_item * 2, nullptr, (int64_t)m->ld_item, 0, k, 8,
                                   sg.col0, 0};
          }
          kb = sg.k_end;
        }
        g.W = m->wptr("_mlp0.item.weight");
        g.R = ws + w.u_req;
        g.r_f32 = 1;
        g.r_rowmap = (const int32_t*)(ws + w.cand_req) + r0;
        g.r_ld = m->hidden[0];
      } else if (i == 0) {
        input_segments(m, ws, w, g, r0);
      } else {
        g.nseg = 1;
        g.seg[0] = ASeg{ws + w.h[cur], nullptr, (int64_t)in, 0, in, 8, 0, 0};
      }
      g.bias = (const float*)m->wptr("mlp." + std::to_string(i) + ".bias");
      const int nxt = cur == 0 ? 1 : 0;
      g.C = ws + w.h[nxt];
      g.ldc = width;
      g.c_nstride8 = 8;
      g.relu = 1;
      // The last hidden layer takes the output layer into its epilogue when the wide kernel runs
      // it (per-row partials per 64 columns instead of the activations); debug mode keeps the
      // activations for export.
      if (i == L_ - 1 && !m->debug && gemm_fuses_output(g)) {
        g.ow = w_out;
        g.opart = (float*)(ws + w.opart);
        g.opart_ld = mc;
        fused = true;
      }
      e = L(STAGE_MLP_GEMM, [&] { return launch_gemm(g, sp.lowp, s); });
      if (e != hipSuccess) return e;
      cur = nxt;
      in = width;
    }
    m->last_hidden_buf = cur;
    const void* H = ws + w.h[cur];
    e = L(STAGE_DLRM_OUTPUT, [&] {
      if (fused)
        return launch_dlrm_logit((const float*)(ws + w.opart), in / kOutGroup, mc, mc, b_out,
                                 (float*)(ws + w.logits) + r0, out + r0, s);
      return launch_dlrm_output(H, mc, in, w_out, b_out, (float*)(ws + w.logits) + r0, out + r0, sp.lowp, s);
    });
    if (e != hipSuccess) return e;
  }
  return e;
}

extern "C" cvr_status cvr_score(cvr_handle h, const cvr_batch* b, void* workspace, size_t ws_bytes, float* out_scores,
                                void* hip_stream) {
  return cvr::score_call(h, b, workspace, ws_bytes, out_scores, hip_stream);
}

// The scoring call behind cvr_score and the entry points that bring their own workspace.
cvr_status cvr::score_call(cvr_handle h, const cvr_batch* b, void* workspace, size_t ws_bytes, float* out_scores,
                           void* hip_stream) {
  if (!h) return fail(nullptr, CVR_ERR_ARG, "null handle");
  WsPlan plan;
  cvr_status st = check_batch(h, b, workspace, ws_bytes, out_scores, plan);
  if (st != CVR_OK) return st;
  if (h->spec.model == CVR_MODEL_DLRM && h->spec.n_hidden == 0) return fail(h, CVR_ERR_UNSUPPORTED, "DLRM without hidden layers");
  hipStream_t s = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  h->last_ws = ws;
  h->last_plan = plan;
  h->last_R = b->n_requests;
  h->last_n = b->n_candidates;
  h->last_P = b->n_positions;
  h->last_debug = h->debug;
  Launcher L(h, s);
  hipError_t e = run_front(h, b, ws, plan, L, s);
  if (e == hipSuccess && b->n_candidates > 0) {
    if (h->spec.model == CVR_MODEL_DLRM) e = run_dlrm(h, b, ws, plan, out_scores, L, s);
    else e = run_hyformer(h, b, ws, plan, out_scores, L, s);
  }
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return CVR_OK;
}

// ------------------------------------------------------------------ graph replay per batch bucket
void GraphCache::reset() {
  for (GraphEntry& g : entries) {
    for (hipGraphExec_t x : g.exec)
      if (x) (void)hipGraphExecDestroy(x);
    if (g.graph) (void)hipGraphDestroy(g.graph);
  }
  entries.clear();
}

static int64_t round_bucket(int64_t x) {
  if (x < 16) return x;
  int k = 0;
  while ((x >> k) >= 16) ++k;
  return ((x + (int64_t{1} << k) - 1) >> k) << k;  // m * 2^k, 8 <= m <= 16
}

void cvr::bucket_sizes(const cvr_model* m, int64_t R, int64_t n, int64_t ids, int64_t P, int64_t& Rb, int64_t& nb,
                       int64_t& idsb, int64_t& Pb) {
  Rb = round_bucket(R + 1);
  nb = round_bucket(n + 1);
  idsb = round_bucket(ids);
  Pb = m->spec.model == CVR_MODEL_HYFORMER ? round_bucket(P) : 0;
}

GraphPlan cvr::plan_graph(const cvr_model* m, int64_t Rb, int64_t nb, int64_t idsb, int64_t Pb) {
  GraphPlan g;
  g.plan = plan_workspace(m, Rb, nb, Pb);
  size_t off = g.plan.total;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  int64_t bags = 0;
  for (int f = 0; f < m->spec.n_features; ++f) bags += m->feats[f].side == CVR_SIDE_ITEM ? nb : Rb;
  const bool cvrm = m->spec.model == CVR_MODEL_HYFORMER;
  const int tasks = cvrm ? m->spec.n_tasks : 1;
  g.co = take((size_t)(Rb + 1) * 4);
  g.bo = take((size_t)(bags + 1) * 4);
  g.ids = take((size_t)idsb * 4);
  g.so = take(cvrm ? (size_t)m->spec.n_seq * (Rb + 1) * 4 : 0);
  g.scores = take((size_t)nb * tasks * 4);
  g.hdr = take(sizeof(BucketHeader));
  g.total = align256(off);
  return g;
}

static bool bucket_fits(const cvr_model* m, int64_t Rb, int64_t nb, int64_t idsb, int64_t Pb) {
  if (Rb > INT32_MAX || nb > INT32_MAX || idsb > INT32_MAX || Pb > INT32_MAX) return false;
  if (m->spec.model == CVR_MODEL_HYFORMER && (int64_t)m->spec.n_seq * Rb >= (1 << 23)) return false;
  int64_t bags = 0;
  for (int f = 0; f < m->spec.n_features; ++f) bags += m->feats[f].side == CVR_SIDE_ITEM ? nb : Rb;
  return bags < INT32_MAX;
}

extern "C" cvr_status cvr_graph_workspace_bytes(cvr_handle h, int32_t max_requests, int32_t max_candidates,
                                                int64_t max_ids, int64_t max_positions, size_t* bytes) {
  if (!h || !bytes) return fail(h, CVR_ERR_ARG, "null argument");
  if (max_requests < 1 || max_candidates < 0 || max_ids < 0 || max_positions < 0) return fail(h, CVR_ERR_ARG, "bad size");
  int64_t Rb, nb, idsb, Pb;
  bucket_sizes(h, max_requests, max_candidates, max_ids, max_positions, Rb, nb, idsb, Pb);
  if (!bucket_fits(h, Rb, nb, idsb, Pb)) return fail(h, CVR_ERR_ARG, "sizes beyond the int32 limits of the batch layout");
  *bytes = plan_graph(h, Rb, nb, idsb, Pb).total;
  return CVR_OK;
}

extern "C" cvr_status cvr_graph_info(cvr_handle h, int64_t* graphs_held, int64_t* captures) {
  if (!h || !graphs_held || !captures) return fail(h, CVR_ERR_ARG, "null argument");
  *graphs_held = (int64_t)h->graph.entries.size();
  *captures = h->graph.captures;
  return CVR_OK;
}

// Capture one scoring call on the bucket's staging arrays into a graph.
static cvr_status capture_bucket(cvr_model* h, const GraphPlan& gp, const GraphKey& key, const BucketPadParams& pad,
                                 hipStream_t s, GraphEntry& out) {
  char* ws = (char*)key.ws;
  cvr_batch sb{};
  sb.n_requests = key.R;
  sb.n_candidates = key.n;
  sb.n_ids = key.ids;
  sb.n_positions = key.P;
  sb.cand_offsets = (const int32_t*)(ws + gp.co);
  sb.bag_offsets = (const int32_t*)(ws + gp.bo);
  sb.ids = (const int32_t*)(ws + gp.ids);
  if (h->spec.model == CVR_MODEL_HYFORMER) {
    sb.seq_offsets = (const int32_t*)(ws + gp.so);
    sb.seq_ids = pad.sid;  // replaced at run time by the header's pointer (capture_seq_ids_ref)
    h->capture_seq_ids_ref = &((const BucketHeader*)(ws + gp.hdr))->seq_ids;
  }
  float* scores = (float*)(ws + gp.scores);
  const int tasks = h->spec.model == CVR_MODEL_HYFORMER ? h->spec.n_tasks : 1;
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("begin capture: ") + hipGetErrorString(e));
  Launcher L(h, s, false);
  e = run_front(h, &sb, ws, gp.plan, L, s, true);
  if (e == hipSuccess) {
    if (h->spec.model == CVR_MODEL_DLRM) e = run_dlrm(h, &sb, ws, gp.plan, scores, L, s);
    else e = run_hyformer(h, &sb, ws, gp.plan, scores, L, s);
  }
  if (e == hipSuccess)
    e = launch_bucket_copy_out((const BucketHeader*)(ws + gp.hdr), scores, (int64_t)key.n * tasks, s);
  h->capture_seq_ids_ref = nullptr;
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(s, &graph);
  if (e == hipSuccess) e = ec;
  hipGraphExec_t exec[2] = {nullptr, nullptr};
  for (int k = 0; k < 2 && e == hipSuccess; ++k) e = hipGraphInstantiate(&exec[k], graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    for (hipGraphExec_t x : exec)
      if (x) (void)hipGraphExecDestroy(x);
    if (graph) (void)hipGraphDestroy(graph);
    return fail(h, CVR_ERR_HIP, std::string("graph capture failed: ") + hipGetErrorString(e));
  }
  out.key = key;
  out.graph = graph;
  out.exec[0] = exec[0];
  out.exec[1] = exec[1];
  out.last_tok = h->last_tok;
  out.last_attn_tok = h->last_attn_tok;
  out.last_hidden_buf = h->last_hidden_buf;
  out.last_tok_bf16 = h->last_tok_bf16;
  h->graph.captures++;
  return CVR_OK;
}

extern "C" cvr_status cvr_score_graph(cvr_handle h, const cvr_batch* b, void* workspace, size_t ws_bytes,
                                      float* out_scores, void* hip_stream) {
  if (!h) return fail(nullptr, CVR_ERR_ARG, "null handle");
  if (!hip_stream) return fail(h, CVR_ERR_ARG, "graph replay needs a created stream (the null stream cannot be captured)");
  cvr_status st = check_batch_args(h, b, workspace, out_scores);
  if (st != CVR_OK) return st;
  if (h->spec.model == CVR_MODEL_DLRM && h->spec.n_hidden == 0) return fail(h, CVR_ERR_UNSUPPORTED, "DLRM without hidden layers");
  int64_t Rb, nb, idsb, Pb;
  bucket_sizes(h, b->n_requests, b->n_candidates, b->n_ids, b->n_positions, Rb, nb, idsb, Pb);
  if (!bucket_fits(h, Rb, nb, idsb, Pb)) return fail(h, CVR_ERR_ARG, "batch bucket beyond the int32 limits of the batch layout");
  const GraphPlan gp = plan_graph(h, Rb, nb, idsb, Pb);
  if (ws_bytes < gp.total)
    return fail(h, CVR_ERR_WORKSPACE, "workspace too small for this batch's bucket: need " + std::to_string(gp.total) +
                                          " bytes (cvr_graph_workspace_bytes)");
  hipStream_t s = (hipStream_t)hip_stream;
  char* ws = (char*)workspace;
  GraphKey key;
  key.R = (int32_t)Rb;
  key.n = (int32_t)nb;
  key.ids = idsb;
  key.P = Pb;
  key.ws = workspace;
  key.ws_bytes = ws_bytes;
  key.stream = s;
  key.debug = h->debug;
  // the padding kernel's arguments for this call: the caller's batch into the bucket's staging arrays
  BucketPadParams p{};
  p.co = b->cand_offsets;
  p.bo = b->bag_offsets;
  p.ids = b->ids;
  p.so = h->spec.model == CVR_MODEL_HYFORMER ? b->seq_offsets : nullptr;
  p.sid = h->spec.model == CVR_MODEL_HYFORMER ? b->seq_ids : nullptr;
  p.R = b->n_requests;
  p.n = b->n_candidates;
  p.n_ids = b->n_ids;
  p.P = h->spec.model == CVR_MODEL_HYFORMER ? b->n_positions : 0;
  p.S = h->spec.model == CVR_MODEL_HYFORMER ? h->spec.n_seq : 0;
  p.ncols = h->spec.model == CVR_MODEL_HYFORMER ? h->spec.n_seq_cols : 0;
  p.Rb = (int32_t)Rb;
  p.nb = (int32_t)nb;
  p.ids_b = idsb;
  p.Pb = Pb;
  p.nf = h->spec.n_features;
  p.base[0] = p.base_b[0] = 0;
  for (int f = 0; f < p.nf; ++f) {
    const bool item = h->feats[f].side == CVR_SIDE_ITEM;
    p.base[f + 1] = p.base[f] + (item ? b->n_candidates : b->n_requests);
    p.base_b[f + 1] = p.base_b[f] + (item ? nb : Rb);
  }
  p.total_bags = p.base[p.nf];
  p.total_bags_b = p.base_b[p.nf];
  p.co_b = (int32_t*)(ws + gp.co);
  p.bo_b = (int32_t*)(ws + gp.bo);
  p.ids_bk = (int32_t*)(ws + gp.ids);
  p.so_b = (int32_t*)(ws + gp.so);
  p.hdr = (BucketHeader*)(ws + gp.hdr);
  p.out = out_scores;
  p.tasks = h->spec.model == CVR_MODEL_HYFORMER ? h->spec.n_tasks : 1;
  GraphCache& gc = h->graph;
  gc.calls++;
  GraphEntry* g = nullptr;
  for (GraphEntry& e : gc.entries)
    if (e.key == key) g = &e;
  if (!g) {
    if ((int)gc.entries.size() >= GraphCache::kMaxGraphs) {  // release the least recently used
      size_t lru = 0;
      for (size_t i = 1; i < gc.entries.size(); ++i)
        if (gc.entries[i].used < gc.entries[lru].used) lru = i;
      for (hipGraphExec_t x : gc.entries[lru].exec)
        if (x) (void)hipGraphExecDestroy(x);
      if (gc.entries[lru].graph) (void)hipGraphDestroy(gc.entries[lru].graph);
      gc.entries.erase(gc.entries.begin() + (long)lru);
    }
    GraphEntry fresh;
    st = capture_bucket(h, gp, key, p, s, fresh);
    if (st != CVR_OK) return st;
    gc.entries.push_back(fresh);
    g = &gc.entries.back();
  }
  g->used = gc.calls;
  // an ordinary launch ahead of the replay (updating a node of the executable graph instead was
  // measured to hold the host until the device had caught up)
  hipError_t e = launch_bucket_pad(p, s);
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("bucket padding: ") + hipGetErrorString(e));
  e = hipGraphLaunch(g->exec[g->next], s);
  g->next ^= 1;
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("graph launch: ") + hipGetErrorString(e));

  // the handle now describes the replayed call: the bucket's padded batch
  h->last_ws = ws;
  h->last_plan = gp.plan;
  h->last_R = Rb;
  h->last_n = nb;
  h->last_P = Pb;
  h->last_debug = g->key.debug;
  h->last_tok = g->last_tok;
  h->last_attn_tok = g->last_attn_tok;
  h->last_hidden_buf = g->last_hidden_buf;
  h->last_tok_bf16 = g->last_tok_bf16;
  return CVR_OK;
}

extern "C" cvr_status cvr_sync_status(cvr_handle h, void* hip_stream) {
  if (!h) return fail(nullptr, CVR_ERR_ARG, "null handle");
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("stream sync: ") + hipGetErrorString(e));
  if (!h->last_ws) return CVR_OK;
  // the status word and the expand launch's per-block words, which sit right after it
  const WsPlan& lp = h->last_plan;
  std::vector<int32_t> words((lp.expand_err - lp.flag) / 4 + (size_t)lp.expand_blocks);
  e = hipMemcpy(words.data(), h->last_ws + lp.flag, words.size() * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("reading status: ") + hipGetErrorString(e));
  int32_t flag = words[0];
  for (int64_t b = 0; b < lp.expand_blocks; ++b) flag |= words[(lp.expand_err - lp.flag) / 4 + b];
  if (flag) {
    std::string why = "device check failed:";
    if (flag & ERRF_CAND_OFFSETS) why += " cand_offsets malformed;";
    if (flag & ERRF_BAG_OFFSETS) why += " bag_offsets malformed;";
    if (flag & ERRF_ID_RANGE) why += " id outside its table;";
    if (flag & ERRF_SEQ_OFFSETS) why += " seq_offsets malformed;";
    if (flag & ERRF_SEQ_ID_RANGE) why += " sequence id outside its table;";
    return fail(h, CVR_ERR_RANGE, why);
  }
  return CVR_OK;
}

// ------------------------------------------------------------------ debug export

extern "C" cvr_status cvr_set_option(cvr_handle h, int32_t option, int64_t value) {
  if (!h) return fail(nullptr, CVR_ERR_ARG, "null handle");
  switch (option) {
    case CVR_OPT_DLRM_PASS_ROWS:
      if (value < -1 || value > INT32_MAX) return fail(h, CVR_ERR_ARG, "pass rows must be -1, 0 or a count");
      h->pass_rows = value;
      break;
    case CVR_OPT_TOK_SHARE:
      if (value < -1 || value > 1) return fail(h, CVR_ERR_ARG, "tokenizer sharing must be -1, 0 or 1");
      h->opt_tok_share = (int)value;
      break;
    case CVR_OPT_ATTN_MQ:
      if (value < -1 || value > 1) return fail(h, CVR_ERR_ARG, "attention form must be -1, 0 or 1");
      h->opt_attn_mq = (int)value;
      break;
    case CVR_OPT_DLRM_USER_BLOCK:
      if (value < -1 || value > 1) return fail(h, CVR_ERR_ARG, "user block must be -1, 0 or 1");
      if (value == 1 && !h->dlrm_split)
        return fail(h, CVR_ERR_UNSUPPORTED, "the user block needs a DLRM spec with both sides, runs of 32 columns");
      h->opt_user_block = (int)value;
      break;
    case CVR_OPT_HEADS_FUSED:
      if (value < -1 || value > 1) return fail(h, CVR_ERR_ARG, "fused heads must be -1, 0 or 1");
      if (value == 1 && (h->spec.model != CVR_MODEL_HYFORMER || !heads_fusable(h->spec.expert_dim, h->spec.head_hidden, h->spec.n_experts, h->spec.n_tasks)))
        return fail(h, CVR_ERR_UNSUPPORTED, "fused heads need a CVR spec with expert and head widths of at most 256, at most 4 experts and 4 tasks");
      h->opt_heads_fused = (int)value;
      break;
    case CVR_OPT_STATE_STREAM:
      if (value < -1 || value > 1) return fail(h, CVR_ERR_ARG, "state streaming must be -1, 0 or 1");
      h->opt_state_stream = (int)value;
      break;
    default: return fail(h, CVR_ERR_ARG, "unknown option");
  }
  h->graph.reset();  // a captured graph baked in the previous choice
  return CVR_OK;
}

extern "C" cvr_status cvr_set_debug(cvr_handle h, int32_t debug) {
  if (!h) return fail(nullptr, CVR_ERR_ARG, "null handle");
  h->debug = debug ? 1 : 0;
  return CVR_OK;
}

extern "C" cvr_status cvr_debug_export(cvr_handle h, int32_t what, void* dst, size_t dst_bytes, size_t* written,
                                       void* hip_stream) {
  if (!h || !dst) return fail(h, CVR_ERR_ARG, "null argument");
  if (!h->last_ws) return fail(h, CVR_ERR_ARG, "nothing scored yet");
  const WsPlan& w = h->last_plan;
  const cvr_spec& sp = h->spec;
  const size_t R = h->last_R, n = h->last_n, P = h->last_P;
  size_t off = 0, bytes = 0;
  const bool cvr = sp.model == CVR_MODEL_HYFORMER;
  const size_t d = sp.d, S = sp.n_seq, T = sp.n_tokens + sp.n_seq;
  switch (what) {
    case CVR_DBG_CAND_REQ: off = w.cand_req; bytes = n * 4; break;
    case CVR_DBG_POOLED:
      if (!h->last_debug) return fail(h, CVR_ERR_ARG, "pooled values need cvr_set_debug(1) before scoring");
      off = w.pooled; bytes = w.pooled_bytes; break;
    case CVR_DBG_INPUT_REQ: off = w.x_req; bytes = R * h->ld_req * 2; break;
    case CVR_DBG_INPUT_ITEM: off = w.x_item; bytes = n * h->ld_item * 2; break;
    case CVR_DBG_LOGITS: off = w.logits; bytes = n * (cvr ? sp.n_tasks : 1) * 4; break;
    case CVR_DBG_HSEQ: if (!cvr) return fail(h, CVR_ERR_ARG, "CVR only"); off = w.hseq; bytes = P * d * 2; break;
    case CVR_DBG_SEQ_POOL: if (!cvr) return fail(h, CVR_ERR_ARG, "CVR only"); off = w.seq_pool; bytes = S * R * d * 4; break;
    case CVR_DBG_TOKENS:
      if (!cvr) return fail(h, CVR_ERR_ARG, "CVR only");
      if (h->last_tok_bf16)
        return fail(h, CVR_ERR_ARG, "the token matrix is kept in fp32 only with cvr_set_debug(1) before scoring (otherwise "
                                    "the last layer writes it as bf16 for the expert GEMM)");
      off = w.tok[h->last_tok]; bytes = n * T * d * 4; break;
    case CVR_DBG_QUERY: if (!cvr) return fail(h, CVR_ERR_ARG, "CVR only"); off = w.query; bytes = S * n * d * 4; break;
    case CVR_DBG_ATTN: if (!cvr) return fail(h, CVR_ERR_ARG, "CVR only"); off = w.tok[h->last_attn_tok]; bytes = n * T * d * 4; break;
    case CVR_DBG_HIDDEN:
      if (cvr || sp.n_hidden == 0) return fail(h, CVR_ERR_ARG, "DLRM with hidden layers only");
      if (!h->last_debug)
        return fail(h, CVR_ERR_ARG, "hidden activations need cvr_set_debug(1) before scoring (otherwise the last "
                                    "hidden layer may be fused into the output layer)");
      off = w.h[h->last_hidden_buf]; bytes = n * h->hidden[sp.n_hidden - 1] * 2; break;
    case CVR_DBG_EPNET:
      if (!cvr || sp.epnet_hidden == 0) return fail(h, CVR_ERR_ARG, "CVR model with EPNet only");
      off = w.x_ep; bytes = n * h->e_dim * 2; break;
    default: return fail(h, CVR_ERR_ARG, "unknown export");
  }
  if (dst_bytes < bytes) return fail(h, CVR_ERR_ARG, "destination too small: need " + std::to_string(bytes));
  if (bytes) {
    hipError_t e = hipMemcpyAsync(dst, h->last_ws + off, bytes, hipMemcpyDeviceToDevice, (hipStream_t)hip_stream);
    if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("export copy: ") + hipGetErrorString(e));
  }
  if (written) *written = bytes;
  return CVR_OK;
}

// ------------------------------------------------------------------ misc

// ------------------------------------------------------------------ HBM hot-row cache

extern "C" cvr_status cvr_cache_state_bytes(int64_t sets, int32_t ways, int32_t dim, size_t* bytes) {
  if (!bytes) return fail(nullptr, CVR_ERR_ARG, "bytes is null");
  if (sets < 1 || ways < 1 || ways > kCacheMaxWays || sets * ways >= INT32_MAX || dim < 4 || dim % 4)
    return fail(nullptr, CVR_ERR_ARG, "bad cache shape");
  *bytes = cache_layout(sets, ways, dim).total;
  return CVR_OK;
}

static const cvr_model::Cache* find_cache(const cvr_model* m, int32_t table) {
  for (const auto& c : m->caches)
    if (c.table == table) return &c;
  return nullptr;
}

extern "C" cvr_status cvr_cache_attach(cvr_handle h, int32_t table, int64_t sets, int32_t ways, void* state,
                                       size_t state_bytes, void* hip_stream) {
  if (!h) return fail(nullptr, CVR_ERR_ARG, "null handle");
  if (table < 0 || table >= (int32_t)h->tables.size()) return fail(h, CVR_ERR_ARG, "table index out of range");
  const int32_t dim = h->tables[table].dim;
  if (sets < 1 || ways < 1 || ways > std::min(kCacheMaxWays, dim / 4) || sets * ways >= INT32_MAX)
    return fail(h, CVR_ERR_ARG, "cache shape: need 1 <= ways <= min(16, dim/4), sets >= 1, sets*ways < 2^31");
  bool used = false;
  for (int f = 0; f < h->spec.n_features; ++f) used |= h->spec.features[f].table == table;
  if (!used) return fail(h, CVR_ERR_ARG, "no feature reads this table");
  for (int32_t t : h->seq_tables)
    if (t == table) return fail(h, CVR_ERR_UNSUPPORTED, "sequence-column tables cannot be cached");
  if (find_cache(h, table)) return fail(h, CVR_ERR_ARG, "table already has a cache");
  if ((int)h->caches.size() >= kMaxCaches) return fail(h, CVR_ERR_UNSUPPORTED, "at most 4 caches per model");
  if (!state || ((uintptr_t)state & 255)) return fail(h, CVR_ERR_ARG, "state must be non-null and 256-byte aligned");
  const CacheLayout l = cache_layout(sets, ways, dim);
  if (state_bytes < l.total) return fail(h, CVR_ERR_WORKSPACE, "cache state too small");
  // tables[].data already holds the device-side address (cvr_create translates host memory).
  cvr_model::Cache c{table, sets, ways, (char*)state, h->tables[table].data};
  hipError_t e = launch_cache_init(gather_cache(c, dim), (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("cache init: ") + hipGetErrorString(e));
  h->caches.push_back(c);
  h->graph.reset();
  return CVR_OK;
}

extern "C" cvr_status cvr_cache_stats(cvr_handle h, int32_t table, int64_t* counters, void* hip_stream) {
  if (!h || !counters) return fail(h, CVR_ERR_ARG, "null argument");
  const cvr_model::Cache* c = find_cache(h, table);
  if (!c) return fail(h, CVR_ERR_ARG, "table has no cache");
  unsigned long long v[CACHE_NCOUNTERS][kCacheCounterSlots];
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e = hipMemcpyAsync(v, ((CacheHeader*)c->state)->counters, sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("cache stats: ") + hipGetErrorString(e));
  for (int i = 0; i < CACHE_NCOUNTERS; ++i) {
    unsigned long long sum = 0;
    for (int k = 0; k < kCacheCounterSlots; ++k) sum += v[i][k];
    counters[i] = (int64_t)sum;
  }
  return CVR_OK;
}

extern "C" cvr_status cvr_cache_export(cvr_handle h, int32_t table, int32_t* tags, int32_t* stamps, void* hip_stream) {
  if (!h || !tags || !stamps) return fail(h, CVR_ERR_ARG, "null argument");
  const cvr_model::Cache* c = find_cache(h, table);
  if (!c) return fail(h, CVR_ERR_ARG, "table has no cache");
  const CacheLayout l = cache_layout(c->sets, c->ways, h->tables[table].dim);
  const size_t bytes = (size_t)c->sets * c->ways * 4;
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e = hipMemcpyAsync(tags, c->state + l.tags, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(stamps, c->state + l.stamps, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(h, CVR_ERR_HIP, std::string("cache export: ") + hipGetErrorString(e));
  return CVR_OK;
}

extern "C" cvr_status cvr_fill_table(float* table, int64_t rows, int32_t dim, uint64_t seed, double halfwidth,
                                     void* hip_stream) {
  if (!table || ((uintptr_t)table & 15)) return fail(nullptr, CVR_ERR_ARG, "table must be non-null and 16-byte aligned");
  if (rows <= 0 || dim <= 0 || dim % 4) return fail(nullptr, CVR_ERR_ARG, "rows > 0 and dim a positive multiple of 4 required");
  if (!(halfwidth > 0.0) || !std::isfinite(halfwidth)) return fail(nullptr, CVR_ERR_ARG, "halfwidth must be positive");
  const double step = (2.0 * halfwidth) / 16777216.0;
  hipError_t e = launch_fill_table(table, rows * (int64_t)dim, seed, step, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(nullptr, CVR_ERR_HIP, std::string("fill: ") + hipGetErrorString(e));
  return CVR_OK;
}

extern "C" const char* cvr_last_error(cvr_handle h) { return h ? h->err.c_str() : g_last_error.c_str(); }

extern "C" const char* cvr_status_string(cvr_status s) {
  switch (s) {
    case CVR_OK: return "ok";
    case CVR_ERR_ARG: return "invalid argument";
    case CVR_ERR_SPEC: return "invalid spec or weights";
    case CVR_ERR_RANGE: return "id or offset out of range (device check)";
    case CVR_ERR_WORKSPACE: return "workspace or arena too small";
    case CVR_ERR_HIP: return "HIP runtime error";
    case CVR_ERR_UNSUPPORTED: return "unsupported by the kernels";
  }
  return "unknown status";
}

extern "C" void cvr_destroy(cvr_handle h) {
  if (!h) return;
  h->timing.reset();
  h->graph.reset();
  delete h;
}
