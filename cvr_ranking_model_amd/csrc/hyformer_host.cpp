// Launch sequence of the HyFormer-style CVR model (steps B2-B11), after the shared
// expand and gather-pool front.
//
// Token matrices live in two ping-pong buffers of [n][T][d] fp32 (T = N + S tokens); every
// GEMM that reads them rounds its input rows to bf16 as it loads them:
//   tokenize GEMM  -> rows 0..N-1 of buffer `cur`              (B2)
//   SwiGLU + pool  -> H [positions][d], pooled means [S][R][d]   (B3-B5, once per request)
//   per layer l:
//     query GEMM (grouped over sequences) <- rows 0..N-1 of `cur` and the pooled mean (B6)
//     attention                           -> rows N..N+S-1 of `cur`                     (B7)
//     token mixer: one fused kernel for 16 tokens x 128 (heads of 8, FFN 128-256-128) reads
//     the Split layout of `cur` and writes Y + FFN in the Revert layout into the other
//     buffer; other shapes take mixer fc1 / fc2 as grouped GEMMs with the same addressing (B8)
//     the other buffer becomes `cur`: its rows 0..N-1 are the next layer's tokens       (B9)
//   expert GEMM, gates + mixture, head fc1 GEMM, head output + sigmoid                  (B10-B11)
#include <hip/hip_runtime.h>

#include <string>

#include "kernels.h"
#include "model.h"

using namespace cvr;

// Element stride between parameters fmt(0), fmt(1), ... in the arena, or -1 if not uniform.
template <typename F>
static int64_t group_stride(const cvr_model* m, F&& fmt, int count, int elem_bytes) {
  if (count <= 1) return 0;
  const int64_t st = (int64_t)m->w[m->widx.at(fmt(1))].off - (int64_t)m->w[m->widx.at(fmt(0))].off;
  for (int i = 2; i < count; ++i)
    if ((int64_t)m->w[m->widx.at(fmt(i))].off - (int64_t)m->w[m->widx.at(fmt(i - 1))].off != st) return -1;
  return st % elem_bytes ? -1 : st / elem_bytes;
}

static std::string S_(int i) { return std::to_string(i); }

hipError_t run_hyformer(cvr_model* m, const cvr_batch* b, char* ws, const WsPlan& w, float* out, Launcher& L,
                        hipStream_t s) {
  const cvr_spec& sp = m->spec;
  const int R = b->n_requests, n = b->n_candidates, S = sp.n_seq, d = sp.d, N = sp.n_tokens, T = N + S;
  const int H = sp.mixer_heads, mh = sp.mixer_hidden, E = sp.n_experts, ed = sp.expert_dim, K = sp.n_tasks;
  const int hh = sp.head_hidden;
  const int64_t P = b->n_positions;
  const int lowp = CVR_LOWP_BF16;
  char* tok[2] = {ws + w.tok[0], ws + w.tok[1]};
  const int32_t* cand_req = (const int32_t*)(ws + w.cand_req);
  int32_t* flag = (int32_t*)(ws + w.flag);
  hipError_t e;

  // ---- EPNet (optional): e' = e * 2 sigmoid(W2 ReLU(W1 [e_domain, e] + b1) + b2), written as the
  // tokenizer's bf16 input.  Gate input: the scenario columns, then every input run, all read in
  // place (request-side runs through the candidate -> request map).
  const bool ep = sp.epnet_hidden > 0;
  if (ep) {
    GemmParams g{};
    g.M = n;
    g.N = sp.epnet_hidden;
    g.K = m->D_dom + m->e_dim;
    g.groups = 1;
    for (const InputSeg& sg : m->dom_segs)
      g.seg[g.nseg++] = ASeg{ws + w.x_req, cand_req, (int64_t)m->ld_req, 0, sg.k_end, 8, sg.col0, 0};
    for (const InputSeg& sg : m->segs)
      g.seg[g.nseg++] = ASeg{ws + (sg.item ? w.x_item : w.x_req), sg.item ? nullptr : cand_req,
                             (int64_t)(sg.item ? m->ld_item : m->ld_req), 0, m->D_dom + sg.k_end, 8, sg.col0, 0};
    g.W = m->wptr("epnet.fc1.weight");
    g.bias = (const float*)m->wptr("epnet.fc1.bias");
    g.C = ws + w.ep_h;
    g.ldc = sp.epnet_hidden;
    g.c_nstride8 = 8;
    g.relu = 1;
    e = L(STAGE_EPNET, [&] { return launch_gemm(g, lowp, s); });
    if (e != hipSuccess) return e;
    GemmParams g2{};
    g2.M = n;
    g2.N = m->e_dim;
    g2.K = sp.epnet_hidden;
    g2.groups = 1;
    g2.nseg = 1;
    g2.seg[0] = ASeg{ws + w.ep_h, nullptr, (int64_t)sp.epnet_hidden, 0, sp.epnet_hidden, 8, 0, 0};
    g2.W = m->wptr("epnet.fc2.weight");
    g2.bias = (const float*)m->wptr("epnet.fc2.bias");
    g2.C = ws + w.ep_g;
    g2.ldc = m->e_dim;
    g2.c_nstride8 = 8;
    g2.out_f32 = 1;
    e = L(STAGE_EPNET, [&] { return launch_gemm(g2, lowp, s); });
    if (e != hipSuccess) return e;
    EpnetParams ap{};
    ap.n = n;
    ap.D = m->e_dim;
    ap.g = (const float*)(ws + w.ep_g);
    ap.x_req = (const __bf16*)(ws + w.x_req);
    ap.x_item = (const __bf16*)(ws + w.x_item);
    ap.ld_req = m->ld_req;
    ap.ld_item = m->ld_item;
    ap.cand_req = cand_req;
    int kb = 0;
    for (const InputSeg& sg : m->segs) {
      ap.run_k0[ap.nruns] = kb;
      ap.run_col0[ap.nruns] = sg.col0;
      ap.run_item[ap.nruns] = sg.item ? 1 : 0;
      ap.nruns++;
      kb = sg.k_end;
    }
    ap.out = (__bf16*)(ws + w.x_ep);
    e = L(STAGE_EPNET, [&] { return launch_epnet_apply(ap, s); });
    if (e != hipSuccess) return e;
  }

  // ---- B2: tokenization, X = E W_tok^T + b into token rows 0..N-1.  When requests carry several
  // candidates, the request-side columns are multiplied once per request (U = E_req W_req^T)
  // and every candidate adds its request's row of U to its item-side product.
  bool share = m->tok_split && (m->opt_tok_share < 0 ? (int64_t)n >= 4 * (int64_t)R : m->opt_tok_share != 0);
  if (!share) {
    GemmParams g{};
    g.M = n;
    g.N = N * d;
    g.K = m->e_dim;
    g.groups = 1;
    if (ep) {
      g.nseg = 1;
      g.seg[0] = ASeg{ws + w.x_ep, nullptr, (int64_t)m->e_dim, 0, m->e_dim, 8, 0, 0};
    } else {
      g.nseg = (int)m->segs.size();
      for (size_t i = 0; i < m->segs.size(); ++i) {
        const InputSeg& sg = m->segs[i];
        g.seg[i] = ASeg{ws + (sg.item ? w.x_item : w.x_req), sg.item ? nullptr : cand_req,
                        (int64_t)(sg.item ? m->ld_item : m->ld_req), 0, sg.k_end, 8, sg.col0, 0};
      }
    }
    g.W = m->wptr("tok.weight");
    g.bias = (const float*)m->wptr("tok.bias");
    g.C = tok[0];
    g.ldc = (int64_t)T * d;
    g.c_nstride8 = 8;
    g.out_f32 = 1;
    g.C2 = ws + w.xq;  // the first layer's query input
    g.ldc2 = (int64_t)N * d;
    e = L(STAGE_TOKENIZE_GEMM, [&] { return launch_gemm(g, lowp, s); });
    if (e != hipSuccess) return e;
  } else {
    for (int side = 0; side < 2; ++side) {  // 0: request side (M = R), 1: item side (M = n)
      const bool item = side == 1;
      GemmParams g{};
      g.M = item ? n : R;
      g.N = N * d;
      g.K = item ? m->D_item : m->D_req;
      g.groups = 1;
      int kb = 0, k = 0;
      for (const InputSeg& sg : m->segs) {
        if (sg.item == item) {
          k += sg.k_end - kb;
          g.seg[g.nseg++] = ASeg{ws + (item ? w.x_item : w.x_req), nullptr,
                                 (int64_t)(item ? m->ld_item : m->ld_req), 0, k, 8, sg.col0, 0};
        }
        kb = sg.k_end;
      }
      g.W = m->wptr(item ? "_tok.item.weight" : "_tok.req.weight");
      g.C = item ? tok[0] : ws + w.tok_req;
      g.ldc = item ? (int64_t)T * d : (int64_t)N * d;
      g.c_nstride8 = 8;
      g.out_f32 = 1;
      if (item) {
        g.bias = (const float*)m->wptr("tok.bias");
        g.R = ws + w.tok_req;
        g.r_f32 = 1;
        g.r_rowmap = cand_req;
        g.r_ld = (int64_t)N * d;
        g.C2 = ws + w.xq;  // the first layer's query input
        g.ldc2 = (int64_t)N * d;
      }
      e = L(STAGE_TOKENIZE_GEMM, [&] { return launch_gemm(g, lowp, s); });
      if (e != hipSuccess) return e;
    }
  }

  // ---- B3-B5: sequence encoding and mean pools (per request)
  // encoded states larger than the last-level cache go out and come back with nontemporal hints
  const bool stream_states = m->opt_state_stream < 0 ? seq_states_stream(P) : m->opt_state_stream != 0;
  int32_t* chunk_off = (int32_t*)(ws + w.chunk_off);
  // every segment adds at most one partial chunk; the workspace holds this many
  const int max_chunks = (int)(P / kSeqChunk) + S * R;
  int2* chunk_desc = (int2*)(ws + w.chunk_desc);
  if (!seq_plan_in_front(S, R)) {  // else the expand launch made the plan
    e = L(STAGE_SEQ_CHUNKS, [&] { return launch_chunk_table(b->seq_offsets, R, S, P, chunk_off, chunk_desc, s); });
    if (e != hipSuccess) return e;
  }
  {
    SwigluParams p{};
    p.seq_offsets = b->seq_offsets;
    p.R = R;
    p.S = S;
    p.n_positions = P;
    p.seq_ids = b->seq_ids;
    p.seq_ids_ref = m->capture_seq_ids_ref;  // bucket replay: the caller's array, named per call
    p.ncols = sp.n_seq_cols;
    int col = 0;
    for (int c = 0; c < sp.n_seq_cols; ++c) {
      const cvr_table& t = m->tables[m->seq_tables[c]];
      p.col_off[c] = col;
      p.col_dim[c] = t.dim;
      p.col_rows[c] = t.rows;
      p.col_table[c] = t.data;
      col += t.dim;
    }
    p.chunk_off = chunk_off;
    p.desc = chunk_desc;
    p.max_chunks = max_chunks;
    p.Wgu = (const __bf16*)m->wptr("seq.0.gate.weight");
    p.wgu_gstride = group_stride(m, [](int i) { return "seq." + S_(i) + ".gate.weight"; }, S, 2);
    p.bgu = (const float*)m->wptr("seq.0.gate.bias");
    p.bgu_gstride = group_stride(m, [](int i) { return "seq." + S_(i) + ".gate.bias"; }, S, 4);
    p.Wd = (const __bf16*)m->wptr("seq.0.down.weight");
    p.wd_gstride = group_stride(m, [](int i) { return "seq." + S_(i) + ".down.weight"; }, S, 2);
    p.bd = (const float*)m->wptr("seq.0.down.bias");
    p.bd_gstride = group_stride(m, [](int i) { return "seq." + S_(i) + ".down.bias"; }, S, 4);
    if (p.wgu_gstride < 0 || p.bgu_gstride < 0 || p.wd_gstride < 0 || p.bd_gstride < 0) return hipErrorInvalidValue;
    p.clamp = sp.clamp;
    p.H = (__bf16*)(ws + w.hseq);
    p.part = (float*)(ws + w.pool_part);
    p.flag = flag;
    p.nt = stream_states;
    e = L(STAGE_SWIGLU, [&] { return launch_swiglu(p, max_chunks, s); });
    if (e != hipSuccess) return e;
  }
  e = L(STAGE_SEQ_POOL, [&] {
    return launch_seq_pool((const float*)(ws + w.pool_part), chunk_off, b->seq_offsets, R, S, P, max_chunks,
                           (float*)(ws + w.seq_pool), (__bf16*)(ws + w.pool_bf), stream_states, s);
  });
  if (e != hipSuccess) return e;

  // ---- B6-B9: stacked interaction layers
  int cur = 0;
  bool last_bf16 = false;
  for (int l = 0; l < sp.n_layers; ++l) {
    const std::string Lp = "layer." + S_(l);
    {
      GemmParams g{};
      g.M = n;
      g.N = d;
      g.K = (N + 1) * d;
      g.groups = S;
      g.nseg = 2;
      // the first layer reads [X, pool] from the bf16 copies the tokenizer and the pool kernel
      // wrote (the same values the fp32 sources round to on loading, at half the bytes); later
      // layers read the mixer's fp32 tokens (a bf16 copy from the mixer cost it more than the
      // query GEMM saved)
      if (l == 0) {
        g.seg[0] = ASeg{ws + w.xq, nullptr, (int64_t)N * d, 0, N * d, 8, 0, 0};
        g.seg[1] = ASeg{ws + w.pool_bf, cand_req, d, (int64_t)R * d, (N + 1) * d, 8, 0, 0};
      } else {
        g.seg[0] = ASeg{tok[cur], nullptr, (int64_t)T * d, 0, N * d, 8, 0, 1};
        g.seg[1] = ASeg{ws + w.seq_pool, cand_req, d, (int64_t)R * d, (N + 1) * d, 8, 0, 1};
      }
      g.W = m->wptr(Lp + ".query.0.weight");
      g.w_gstride = group_stride(m, [&](int i) { return Lp + ".query." + S_(i) + ".weight"; }, S, 2);
      g.bias = (const float*)m->wptr(Lp + ".query.0.bias");
      g.bias_gstride = group_stride(m, [&](int i) { return Lp + ".query." + S_(i) + ".bias"; }, S, 4);
      if (g.w_gstride < 0 || g.bias_gstride < 0) return hipErrorInvalidValue;
      g.C = ws + w.query;
      g.ldc = d;
      g.c_gstride = (int64_t)n * d;
      g.c_nstride8 = 8;
      g.out_f32 = 1;
      // many candidates per request: the token rows stay cache-resident, and one tile per row
      // block and query reads them once instead of once per 64 columns
      g.full_n = (int64_t)n >= 4 * (int64_t)R;
      e = L(STAGE_QUERY_GEMM, [&] { return launch_gemm(g, lowp, s); });
      if (e != hipSuccess) return e;
    }
    {
      AttnParams a{};
      a.H = (const __bf16*)(ws + w.hseq);
      a.seq_offsets = b->seq_offsets;
      a.R = R;
      a.S = S;
      a.n_positions = P;
      a.q = (const float*)(ws + w.query);
      a.cand_req = cand_req;
      a.n = n;
      a.inv_tau = 1.0f / sp.tau;
      a.Y = (float*)tok[cur];
      a.T = T;
      a.N = N;
      a.mq = m->opt_attn_mq < 0 ? attention_many_candidates(n, R) : m->opt_attn_mq != 0;
      // nontemporal loads from the second layer on: the first layer reads the states right after
      // the encoder wrote them, and there plain loads measured faster (C4: 607 against 643 us;
      // the second layer 522 us with the hint)
      a.nt = stream_states && l > 0;
      e = L(STAGE_ATTENTION, [&] { return launch_attention(a, s); });
      if (e != hipSuccess) return e;
    }
    const int mw = T * d / H;  // mixed-token width; one 8-wide chunk per token
    if (token_mix_supported(T, d, H, mh)) {
      TokenMixParams t{};
      t.Y = (const float*)tok[cur];
      t.Z = (float*)tok[1 - cur];
      // The last layer's tokens feed only the expert GEMM, which rounds them to bf16 as it loads
      // them: written as bf16 they take half the bytes and give the same products.  Debug runs
      // keep fp32 so that the token matrix can be exported.
      if (l == sp.n_layers - 1 && !m->debug) t.Zb = (__bf16*)tok[1 - cur];
      last_bf16 = t.Zb != nullptr;
      t.n = n;
      t.T = T;
      t.d = d;
      t.H = H;
      t.W1 = (const __bf16*)m->wptr(Lp + ".mix.0.fc1.weight");
      t.w1_gstride = group_stride(m, [&](int i) { return Lp + ".mix." + S_(i) + ".fc1.weight"; }, H, 2);
      t.b1 = (const float*)m->wptr(Lp + ".mix.0.fc1.bias");
      t.b1_gstride = group_stride(m, [&](int i) { return Lp + ".mix." + S_(i) + ".fc1.bias"; }, H, 4);
      t.W2 = (const __bf16*)m->wptr(Lp + ".mix.0.fc2.weight");
      t.w2_gstride = group_stride(m, [&](int i) { return Lp + ".mix." + S_(i) + ".fc2.weight"; }, H, 2);
      t.b2 = (const float*)m->wptr(Lp + ".mix.0.fc2.bias");
      t.b2_gstride = group_stride(m, [&](int i) { return Lp + ".mix." + S_(i) + ".fc2.bias"; }, H, 4);
      if (t.w1_gstride < 0 || t.b1_gstride < 0 || t.w2_gstride < 0 || t.b2_gstride < 0) return hipErrorInvalidValue;
      e = L(STAGE_MIXER_GEMM, [&] { return launch_token_mix(t, s); });
      if (e != hipSuccess) return e;
    } else {
      {
        GemmParams g{};
        g.M = n;
        g.N = mh;
        g.K = mw;
        g.groups = H;
        g.nseg = 1;
        // Split: mixed token h, element t*8 + j = token t, column h*8 + j
        g.seg[0] = ASeg{tok[cur], nullptr, (int64_t)T * d, d / H, mw, d, 0, 1};
        g.W = m->wptr(Lp + ".mix.0.fc1.weight");
        g.w_gstride = group_stride(m, [&](int i) { return Lp + ".mix." + S_(i) + ".fc1.weight"; }, H, 2);
        g.bias = (const float*)m->wptr(Lp + ".mix.0.fc1.bias");
        g.bias_gstride = group_stride(m, [&](int i) { return Lp + ".mix." + S_(i) + ".fc1.bias"; }, H, 4);
        if (g.w_gstride < 0 || g.bias_gstride < 0) return hipErrorInvalidValue;
        g.C = ws + w.mixhid;
        g.ldc = mh;
        g.c_gstride = (int64_t)n * mh;
        g.c_nstride8 = 8;
        g.relu = 1;
        e = L(STAGE_MIXER_GEMM, [&] { return launch_gemm(g, lowp, s); });
        if (e != hipSuccess) return e;
      }
      {
        GemmParams g{};
        g.M = n;
        g.N = mw;
        g.K = mh;
        g.groups = H;
        g.nseg = 1;
        g.seg[0] = ASeg{ws + w.mixhid, nullptr, mh, (int64_t)n * mh, mh, 8, 0, 0};
        g.W = m->wptr(Lp + ".mix.0.fc2.weight");
        g.w_gstride = group_stride(m, [&](int i) { return Lp + ".mix." + S_(i) + ".fc2.weight"; }, H, 2);
        g.bias = (const float*)m->wptr(Lp + ".mix.0.fc2.bias");
        g.bias_gstride = group_stride(m, [&](int i) { return Lp + ".mix." + S_(i) + ".fc2.bias"; }, H, 4);
        if (g.w_gstride < 0 || g.bias_gstride < 0) return hipErrorInvalidValue;
        // Revert + residual: output element t*8 + j of mixed token h lands on token t, column h*8 + j
        g.C = tok[1 - cur];
        g.R = tok[cur];
        g.ldc = (int64_t)T * d;
        g.c_nstride8 = d;
        g.c_gstride = d / H;
        g.out_f32 = 1;
        g.r_f32 = 1;
        e = L(STAGE_MIXER_GEMM, [&] { return launch_gemm(g, lowp, s); });
        if (e != hipSuccess) return e;
      }
    }
    m->last_attn_tok = cur;
    cur = 1 - cur;
  }
  m->last_tok = cur;
  m->last_tok_bf16 = last_bf16;

  // ---- B10: experts and gate logits over the flattened token matrix in one GEMM (the gate
  // rows follow the expert rows in the arena; ReLU on the expert columns only), then the gate
  // softmax and mixture
  int gates = 0;
  int goff[kMaxTasks];
  for (int k = 0; k < K; ++k) {
    goff[k] = gates;
    gates += __builtin_popcount(m->task_mask[k]);
  }
  const int64_t ld = ((int64_t)E * ed + gates + 31) / 32 * 32;  // rows stay 128-byte aligned
  {
    GemmParams g{};
    g.M = n;
    g.N = E * ed + gates;
    g.K = T * d;
    g.groups = 1;
    g.nseg = 1;
    g.seg[0] = ASeg{tok[cur], nullptr, (int64_t)T * d, 0, T * d, 8, 0, last_bf16 ? 0 : 1};
    g.W = m->wptr("ple.expert.0.weight");
    g.bias = (const float*)m->wptr("_ple.bias");
    // the rows must be contiguous: experts back to back, then the gates task by task
    const char* w0 = (const char*)m->wptr("ple.expert.0.weight");
    if (group_stride(m, [](int i) { return "ple.expert." + S_(i) + ".weight"; }, E, 2) != (int64_t)ed * T * d)
      return hipErrorInvalidValue;
    for (int k = 0; k < K; ++k)
      if ((const char*)m->wptr("ple.gate." + S_(k) + ".weight") != w0 + ((int64_t)E * ed + goff[k]) * T * d * 2)
        return hipErrorInvalidValue;
    g.C = ws + w.experts;
    g.ldc = ld;
    g.c_nstride8 = 8;
    g.relu = 1;
    g.relu_end = E * ed;
    g.out_f32 = 1;
    e = L(STAGE_PLE_GEMM, [&] { return launch_gemm(g, lowp, s); });
    if (e != hipSuccess) return e;
  }
  if (m->opt_heads_fused != 0 && heads_fusable(ed, hh, E, K)) {
    // the gate mixture, the heads' two Linears and the sigmoid in one launch
    HeadsParams p{};
    p.g.experts = (const float*)(ws + w.experts);
    p.g.ld = ld;
    p.g.n = n;
    p.g.E = E;
    p.g.K = K;
    p.g.edim = ed;
    p.g.gate0 = E * ed;
    for (int k = 0; k < K; ++k) {
      p.g.goff[k] = goff[k];
      p.g.emask[k] = m->task_mask[k];
      p.b2[k] = (const float*)m->wptr("head." + S_(k) + ".fc2.bias");
    }
    p.W1 = (const __bf16*)m->wptr("head.0.fc1.weight");
    p.w1_stride = group_stride(m, [](int i) { return "head." + S_(i) + ".fc1.weight"; }, K, 2);
    p.b1 = (const float*)m->wptr("head.0.fc1.bias");
    p.b1_stride = group_stride(m, [](int i) { return "head." + S_(i) + ".fc1.bias"; }, K, 4);
    p.hdim = hh;
    p.w2 = (const __bf16*)m->wptr("head.0.fc2.weight");
    p.w2_stride = group_stride(m, [](int i) { return "head." + S_(i) + ".fc2.weight"; }, K, 2);
    if (p.w1_stride < 0 || p.b1_stride < 0 || (K > 1 && p.w2_stride < 0)) return hipErrorInvalidValue;
    p.logits = (float*)(ws + w.logits);
    p.out = out;
    return L(STAGE_HEAD_GEMM, [&] { return launch_heads(p, s); });
  }
  {
    PleGateParams p{};
    p.experts = (const float*)(ws + w.experts);
    p.ld = ld;
    p.n = n;
    p.E = E;
    p.K = K;
    p.edim = ed;
    p.gate0 = E * ed;
    for (int k = 0; k < K; ++k) {
      p.goff[k] = goff[k];
      p.emask[k] = m->task_mask[k];
    }
    p.task_in = (__bf16*)(ws + w.task_in);
    e = L(STAGE_PLE_GATE, [&] { return launch_ple_gate(p, s); });
    if (e != hipSuccess) return e;
  }
  // ---- B11: heads
  {
    GemmParams g{};
    g.M = n;
    g.N = hh;
    g.K = ed;
    g.groups = K;
    g.nseg = 1;
    g.seg[0] = ASeg{ws + w.task_in, nullptr, ed, (int64_t)n * ed, ed, 8, 0, 0};
    g.W = m->wptr("head.0.fc1.weight");
    g.w_gstride = group_stride(m, [](int i) { return "head." + S_(i) + ".fc1.weight"; }, K, 2);
    g.bias = (const float*)m->wptr("head.0.fc1.bias");
    g.bias_gstride = group_stride(m, [](int i) { return "head." + S_(i) + ".fc1.bias"; }, K, 4);
    if (g.w_gstride < 0 || g.bias_gstride < 0) return hipErrorInvalidValue;
    g.C = ws + w.head_hid;
    g.ldc = hh;
    g.c_gstride = (int64_t)n * hh;
    g.c_nstride8 = 8;
    g.relu = 1;
    e = L(STAGE_HEAD_GEMM, [&] { return launch_gemm(g, lowp, s); });
    if (e != hipSuccess) return e;
  }
  {
    HeadOutParams p{};
    p.U = (const __bf16*)(ws + w.head_hid);
    p.n = n;
    p.K = K;
    p.hdim = hh;
    p.w2 = (const __bf16*)m->wptr("head.0.fc2.weight");
    p.w2_stride = group_stride(m, [](int i) { return "head." + S_(i) + ".fc2.weight"; }, K, 2);
    if (K > 1 && p.w2_stride < 0) return hipErrorInvalidValue;
    for (int k = 0; k < K; ++k) p.b2[k] = (const float*)m->wptr("head." + S_(k) + ".fc2.bias");
    p.logits = (float*)(ws + w.logits);
    p.out = out;
    e = L(STAGE_HEAD_OUT, [&] { return launch_head_out(p, s); });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
