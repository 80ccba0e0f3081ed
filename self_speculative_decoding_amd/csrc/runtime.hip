// Runtime behind the C ABI: context, weight table, workspace views, the pass
// driver (prefill / draft / verify), accept + rollback and the decode loops.
//
// One pass = embedding -> layers -> final norm -> LM head -> argmax, with every
// position read from device state (state[0] = committed length n), so the
// plain greedy loop needs no host synchronisation and a speculative cycle
// needs exactly one (the accept result), as the mlx-dflash README's
// "Apple Silicon Optimizations" describe for their engine.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "host.h"
#include "kernels.h"

using namespace ssd;

#define HIPCHK(x)                                                                                    \
  do {                                                                                               \
    hipError_t e_ = (x);                                                                             \
    if (e_ != hipSuccess) return fail(SSD_E_HIP, "%s failed: %s (%s:%d)", #x, hipGetErrorString(e_), \
                                      __FILE__, __LINE__);                                           \
  } while (0)

#define SSDCHK(x)                    \
  do {                               \
    ssd_status s_ = (x);             \
    if (s_ != SSD_OK) return s_;     \
  } while (0)

namespace {

struct LayerW {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm;
  const void *w_gate, *w_up, *w_down;
  const void *router, *eg, *eu, *ed, *sg, *su, *sd;
  bool moe;
  int ffn;
  int feat_slot;   // index in feat_layers, or -1
};

enum { EV_A, EV_B, EV_C, EV_D, EV_N };

struct GraphEntry {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

}  // namespace

struct ssd_ctx {
  ssd_cfg cfg;
  Layout lay;
  hipStream_t stream;
  char* ws;
  size_t esz;
  const void *embed, *final_norm, *lm_head, *fc;
  std::vector<LayerW> L;
  int state = SSD_ST_LOADED;
  int n = 0;            // host copy of the committed length
  int k = 0;            // drafts in the current block
  int head_rows = 0;    // logits rows of the last pass
  int feat_rows = 0;
  int moe_inject = 0;   // rows of injected routing (0 = router)
  int* hbuf = nullptr;  // pinned host scratch
  hipEvent_t ev[EV_N] = {};
  ssd_stats st;
  // decode/draft/verify passes captured as HIP graphs, keyed by their launch shape
  std::map<std::string, GraphEntry> graphs;
  bool use_graphs = true;
  bool capturing = false;
  int cap_part = 0;        // attention partitions of the pass being captured
  bool trace_on = false;   // record the residual after every layer of decode-loop passes
  float* trace = nullptr;
  char* trace_pts = nullptr;   // and the stored operands of every layer (TracePoints)
  TracePoints tp;
  // exit-state reuse of an early-exit draft (SSD_OPT_KVQ): the draft saves
  // each row's residual and sums of squares after its last layer; a verify
  // of that draft starts at the exit layer E from them
  bool kvq_on = false;
  int tile_wg_min = 0;               // SSD_OPT_TILE_GROUPS
  int kvq_E = -1;                    // exit layer of the current draft, -1: none
  float *exit_x = nullptr, *exit_ss = nullptr;
  std::vector<uint8_t> kvq_rest;     // mask running layers E..L-1 only
  std::vector<uint8_t> kvq_mask;     // the current draft's mask
  // sampling (ssd_set_sampling)
  bool smp_set = false;
  float smp_T = 1.f;
  uint64_t smp_seed = 0;
  float* dlog = nullptr;
  int* tout = nullptr;
  SmpBufs smp{};
  // the last decode-loop pass: its tokens (device), rows, and whether it ran every layer
  const int* last_tok = nullptr;
  int last_M = 0;
  bool last_full = false;
  // device views
  float *x, *ss, *logits, *part_o, *part_ml, *cos_t, *sin_t, *amax_v;
  int* amax_i;
  void *xn, *q, *att, *act, *kc, *vc, *tap, *feat;
  void *xn_p = nullptr, *att_p = nullptr, *act_p = nullptr, *tap_p = nullptr;   // fragment-order GEMM inputs
  int *block, *post, *toks, *dstate, *result, *outlog;
  int *tblock, *tpost, *tstate, *tresult, *toutlog;
  float *m_rlogits, *m_gates, *m_slot_out;
  int *m_ids, *m_inject, *m_groups, *m_union;
  float* m_rstd = nullptr;   // MoE: per-token 1/rms of the folded ffn norm
};

namespace {

static_assert(kSmpChunk == SMP_CHUNK && kSmpRows == SMP_ROWS && kSmpCtlBytes == SMP_CTL_BYTES, "sampling scratch");
constexpr int kCtxBucket = 512;   // positions per graph context bucket (multiple of ATT_PT)

inline void* at(ssd_ctx* c, size_t off) { return c->ws + off; }

// positions per KV cache row: max_ctx rounded up to whole attention partitions
inline int kv_stride(const ssd_cfg& c) { return (c.max_ctx + ATT_PT - 1) / ATT_PT * ATT_PT; }
size_t cache_layer_elems(const ssd_cfg& c) { return (size_t)c.n_kv_heads * kv_stride(c) * c.head_dim; }

MoeArgs moe_args(ssd_ctx* c, int l, int M) {
  const ssd_cfg& g = c->cfg;
  const LayerW& w = c->L[l];
  MoeArgs a{};
  a.X = c->xn; a.M = M; a.d = g.d_model; a.E = g.n_experts; a.top_k = g.top_k; a.fe = g.expert_ffn;
  a.n_shared = g.n_shared; a.router = w.router; a.eg = w.eg; a.ed = w.ed;
  a.sg = w.sg; a.sd = w.sd; a.rlogits = c->m_rlogits; a.ids = c->m_ids; a.gates = c->m_gates;
  a.inject = c->moe_inject ? c->m_inject + (size_t)l * c->lay.R * g.top_k : nullptr;
  a.act = c->act; a.slot_out = c->m_slot_out; a.resid = c->x; a.groups = c->m_groups;
  a.union_out = c->m_union + l; a.dedup = g.moe_dedup;
  a.ssw = resid_tile_width(g.d_model);   // the combine's column runs, also without ss_out
  // the ffn norm folded in: X holds bf16(x * ffn_norm gain) and ss the partials
  a.ss_in = c->ss; a.nss = g.d_model / a.ssw; a.eps = g.rms_eps; a.rstd = c->m_rstd;
  return a;
}

// A GEMM of the pass on the context's stream, with the context's grouping
// option for long passes.
hipError_t run_gemm(ssd_ctx* c, int epi, GemmArgs a) {
  a.tile_wg_min = c->tile_wg_min;
  return launch_gemm(c->cfg.dtype, epi, a, c->stream);
}

// bf16 models fold every RMSNorm that feeds a GEMM (QKV, gate/up, the MoE
// router and expert gate/up, LM head) into that GEMM: the residual's producer
// leaves xn = bf16(x * gain) and per-residual-tile sums of squares in ss, and
// the GEMM scales its product by 1/rms.
// Sums-of-squares partials per row: one per column tile of the residual
// GEMMs (resid_tile_width), as every producer writes them.
inline int n_ss(const ssd_cfg& g) { return g.d_model / resid_tile_width(g.d_model); }

void fold_in(ssd_ctx* c, GemmArgs& a, int row0) {
  const int nss = n_ss(c->cfg);
  a.ss_in = c->ss + (size_t)row0 * nss;
  a.nss = nss;
  a.eps = c->cfg.rms_eps;
}

void fold_out(ssd_ctx* c, GemmArgs& a, const void* gain_next) {
  a.ss_out = c->ss;
  a.xg_out = c->xn;
  a.gain_next = gain_next;
}

// Gain of the norm that follows layer l in this pass: attn_norm of the next
// layer that runs, else the final norm.
const void* next_gain(ssd_ctx* c, int l, const uint8_t* skip) {
  for (int j = l + 1; j < c->cfg.n_layers; ++j)
    if (!(skip && skip[j])) return c->L[j].attn_norm;
  return c->final_norm;
}

// Copies rows [0, M) of a pass buffer (rows of `row` bytes) into trace
// point `pt` of layer l (the head input when l == n_layers).
hipError_t trace_point(ssd_ctx* c, int l, int pt, const void* src, int M) {
  const size_t off = (size_t)l * c->tp.layer + (l < c->cfg.n_layers ? c->tp.off[pt] : 0);
  const size_t row = l < c->cfg.n_layers ? c->tp.row[pt] : c->tp.row[0];
  return launch_copy_f32((const float*)src, (float*)(c->trace_pts + off), (int)(M * row / 4), c->stream);
}

// Passes of kFragMinM..kFragRows rows of dense bf16 models keep a
// fragment-order copy of every GEMM input (frag_index): their GEMMs then load
// each A chunk as two 1 KB reads (whole cache lines) instead of 16 rows of 64
// bytes per load, which costs the wide verify blocks most.  The copy holds
// the same values, so results do not change; a function of M only.
inline bool frag_pass(const ssd_ctx* c, int M) { return c->xn_p && M >= kFragMinM && M <= kFragRows; }

// One decoder layer over M rows at positions state[0] + pos_off + r.  fr:
// every producer also writes the fragment-order copy of the next GEMM's
// input and every GEMM reads that copy (frag_pass).
ssd_status layer_forward(ssd_ctx* c, int l, int M, int pos_off, bool feats, const void* gain_next, bool fr) {
  const ssd_cfg& g = c->cfg;
  const LayerW& w = c->L[l];
  const int d = g.d_model, hq = g.n_q_heads, hkv = g.n_kv_heads, hd = g.head_dim;
  const int dt = g.dtype;
  const bool fold = dt == SSD_BF16;
  hipStream_t s = c->stream;
  void* kc = (char*)c->kc + (size_t)l * cache_layer_elems(g) * c->esz;
  void* vc = (char*)c->vc + (size_t)l * cache_layer_elems(g) * c->esz;

  if (!fold) HIPCHK(launch_rmsnorm(dt, c->x, d, w.attn_norm, c->xn, d, d, g.rms_eps, M, s));
  const bool tr = c->trace_on && M <= g.max_block;
  if (tr) HIPCHK(trace_point(c, l, 0, c->xn, M));
  {
    GemmArgs a{};
    a.X = c->xn; a.ldx = d; a.W0 = w.wq; a.W1 = w.wk; a.W2 = w.wv;
    a.Xp = fr ? c->xn_p : nullptr;
    a.n0 = hq * hd; a.n1 = hkv * hd; a.M = M; a.N = (hq + 2 * hkv) * hd; a.K = d;
    a.q = c->q; a.kc = kc; a.vc = vc; a.cos_t = c->cos_t; a.sin_t = c->sin_t;
    a.state = c->dstate; a.pos_off = pos_off; a.hq = hq; a.hkv = hkv; a.hd = hd; a.max_ctx = kv_stride(g);
    if (fold) fold_in(c, a, 0);
    HIPCHK(run_gemm(c, EPI_QKV, a));
  }
  if (tr) HIPCHK(trace_point(c, l, 1, c->q, M));
  {
    AttnArgs a{};
    a.q = c->q; a.kc = kc; a.vc = vc; a.out = c->att; a.part_o = c->part_o; a.part_ml = c->part_ml; a.pstride = c->lay.n_part;
    a.out_p = fr ? c->att_p : nullptr;
    a.state = c->dstate; a.pos_off = pos_off; a.M = M; a.R = c->lay.R;
    a.hq = hq; a.hkv = hkv; a.hd = hd; a.max_ctx = kv_stride(g);
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
    // a captured pass covers the partitions of its context bucket; workgroups
    // past the last row's position store nothing
    const int n_part = c->capturing ? c->cap_part : (c->n + pos_off + M + ATT_PT - 1) / ATT_PT;
    HIPCHK(launch_attention(dt, a, n_part, s));
  }
  if (tr) HIPCHK(trace_point(c, l, 2, c->att, M));
  {
    GemmArgs a{};
    a.X = c->att; a.ldx = hq * hd; a.W0 = w.wo; a.M = M; a.N = d; a.K = hq * hd; a.y = c->x; a.ldy = d;
    a.Xp = fr ? c->att_p : nullptr;
    if (fold) fold_out(c, a, w.ffn_norm);
    a.xg_out_p = fr ? c->xn_p : nullptr;
    HIPCHK(run_gemm(c, EPI_RESID, a));
  }
  if (tr) HIPCHK(trace_point(c, l, 3, c->x, M));
  if (w.moe) {   // bf16 only: the o projection left bf16(x * ffn_norm) and the partials
    if (tr) HIPCHK(trace_point(c, l, 4, c->xn, M));
    MoeArgs a = moe_args(c, l, M);
    a.ss_out = c->ss; a.xg_out = c->xn; a.gain_next = gain_next;
    HIPCHK(launch_moe(dt, a, s));
    if (tr) HIPCHK(launch_copy_f32((const float*)c->act, (float*)(c->trace_pts + (size_t)l * c->tp.layer + c->tp.off[5]),
                                   (int)((size_t)M * (g.top_k + g.n_shared) * g.expert_ffn * c->esz / 4), s));
  } else {
    if (!fold) HIPCHK(launch_rmsnorm(dt, c->x, d, w.ffn_norm, c->xn, d, d, g.rms_eps, M, s));
    if (tr) HIPCHK(trace_point(c, l, 4, c->xn, M));
    GemmArgs a{};
    a.X = c->xn; a.ldx = d; a.W0 = w.w_gate; a.W1 = w.w_up; a.M = M; a.N = w.ffn; a.K = d;
    a.out = c->act; a.ldo = w.ffn;
    a.Xp = fr ? c->xn_p : nullptr;
    a.out_p = fr ? c->act_p : nullptr;
    if (fold) fold_in(c, a, 0);
    HIPCHK(run_gemm(c, EPI_SWIGLU, a));
    if (tr) HIPCHK(trace_point(c, l, 5, c->act, M));
    GemmArgs b{};
    b.X = c->act; b.ldx = w.ffn; b.W0 = w.w_down; b.M = M; b.N = d; b.K = w.ffn; b.y = c->x; b.ldy = d;
    b.Xp = fr ? c->act_p : nullptr;
    if (feats && w.feat_slot >= 0) {
      b.tap = (char*)c->tap + (size_t)w.feat_slot * d * c->esz;
      b.ldtap = g.n_feat * d;
      if (fr) {
        b.tap_p = c->tap_p;
        b.tap_col = w.feat_slot * d;
      }
    }
    if (fold) fold_out(c, b, gain_next);
    b.xg_out_p = fr ? c->xn_p : nullptr;
    HIPCHK(run_gemm(c, EPI_RESID, b));
  }
  if (c->trace_on && M <= g.max_block)
    HIPCHK(launch_copy_f32(c->x, c->trace + (size_t)l * g.max_block * d, M * d, s));
  return SSD_OK;
}

// Exit-state handling of a pass: save_row >= 0 copies the residual (and its
// sums of squares) of rows [0, M) after the pass's last layer to exit-state
// rows [save_row, save_row + M); load starts the pass from exit-state rows
// [0, M) instead of the embedding (the first layer's folded-norm input is
// recomputed from them); head = false skips the final norm and LM head.
struct PassSpec {
  int save_row = -1;
  bool load = false;
  bool head = true;
};

// Full pass: M tokens from d_tok at positions state[0]+pos_off+r through the
// layers with skip[l] == 0 (all when skip is NULL); the head runs on rows
// [head_row0, head_row0+head_rows) and writes argmax to d_arg.
ssd_status run_pass(ssd_ctx* c, const int* d_tok, int M, int pos_off, const uint8_t* skip, int head_row0,
                    int head_rows, int* d_arg, bool feats, const PassSpec& ps = PassSpec()) {
  const ssd_cfg& g = c->cfg;
  const int d = g.d_model, dt = g.dtype;
  const bool fold = dt == SSD_BF16;
  hipStream_t s = c->stream;
  if (c->moe_inject && M > c->moe_inject)
    return fail(SSD_E_ARG, "pass of %d rows but routing was injected for %d", M, c->moe_inject);
  const bool fr = frag_pass(c, M);
  void* xgp = fr ? c->xn_p : nullptr;
  if (ps.load) {
    HIPCHK(launch_copy_f32(c->exit_x, c->x, M * d, s));
    if (fold) {
      HIPCHK(launch_copy_f32(c->exit_ss, c->ss, M * n_ss(g), s));
      HIPCHK(launch_scale_bf16(c->x, next_gain(c, -1, skip), c->xn, d, M, s, xgp));
    }
  } else if (fold) {
    HIPCHK(launch_embed_norm(d_tok, c->embed, c->x, d, M, next_gain(c, -1, skip), c->xn, c->ss, resid_tile_width(d), s,
                             xgp));
  } else {
    HIPCHK(launch_embed(dt, d_tok, c->embed, c->x, d, M, s));
  }
  for (int l = 0; l < g.n_layers; ++l) {
    if (skip && skip[l]) continue;
    SSDCHK(layer_forward(c, l, M, pos_off, feats, next_gain(c, l, skip), fr));
  }
  if (ps.save_row >= 0) {
    HIPCHK(launch_copy_f32(c->x, c->exit_x + (size_t)ps.save_row * d, M * d, s));
    if (fold) HIPCHK(launch_copy_f32(c->ss, c->exit_ss + (size_t)ps.save_row * n_ss(g), M * n_ss(g), s));
  }
  if (head_rows > 0 && ps.head) {
    if (!fold)
      HIPCHK(launch_rmsnorm(dt, c->x + (size_t)head_row0 * d, d, c->final_norm, c->xn, d, d, g.rms_eps, head_rows, s));
    if (c->trace_on && head_row0 == 0 && head_rows <= g.max_block) HIPCHK(trace_point(c, g.n_layers, 0, c->xn, head_rows));
    GemmArgs a{};
    a.X = fold ? (const void*)((const uint16_t*)c->xn + (size_t)head_row0 * d) : c->xn;
    a.ldx = d; a.W0 = c->lm_head; a.M = head_rows; a.N = g.vocab; a.K = d;
    a.Xp = fr && head_row0 == 0 ? c->xn_p : nullptr;
    a.y = c->logits; a.ldy = g.vocab;
    if (dt == SSD_BF16) {
      // the LM head epilogue leaves (max, index) per 16 columns; reduce those
      fold_in(c, a, head_row0);
      a.amax_v = c->amax_v; a.amax_i = c->amax_i;
      HIPCHK(run_gemm(c, EPI_LOGITS, a));
      HIPCHK(launch_argmax_tiles(c->amax_v, c->amax_i, g.vocab / 16, d_arg, head_rows, s));
    } else {
      HIPCHK(run_gemm(c, EPI_F32, a));
      HIPCHK(launch_argmax(c->logits, g.vocab, g.vocab, d_arg, head_rows, s));
    }
    c->head_rows = head_rows;
  }
  if (feats && g.n_feat > 0) {
    GemmArgs a{};
    a.X = c->tap; a.ldx = g.n_feat * d; a.W0 = c->fc; a.M = M; a.N = d; a.K = g.n_feat * d;
    a.Xp = fr ? c->tap_p : nullptr;
    a.out = c->feat; a.ldo = d;
    HIPCHK(run_gemm(c, EPI_STORE, a));
    c->feat_rows = M;
  }
  return SSD_OK;
}

void destroy_graphs(ssd_ctx* c) {
  for (auto& kv : c->graphs) {
    (void)hipGraphExecDestroy(kv.second.exec);
    (void)hipGraphDestroy(kv.second.graph);
  }
  c->graphs.clear();
}

// One decode-loop pass (draft step, verify or plain decode step) with its head
// on all M rows.  Replays a HIP graph captured on first use: every position is
// read from device state, so one graph serves every context length.
ssd_status decode_pass(ssd_ctx* c, const int* tok, int M, int pos_off, const uint8_t* skip, int* arg, bool feats,
                       const PassSpec& ps = PassSpec()) {
  // checked here as well as in run_pass: a replayed graph never re-runs run_pass
  if (c->moe_inject && M > c->moe_inject)
    return fail(SSD_E_ARG, "pass of %d rows but routing was injected for %d", M, c->moe_inject);
  c->last_tok = tok;
  c->last_M = M;
  c->last_full = !ps.load;
  if (skip)
    for (int l = 0; l < c->cfg.n_layers; ++l) c->last_full = c->last_full && !skip[l];
  if (!c->use_graphs) return run_pass(c, tok, M, pos_off, skip, 0, M, arg, feats, ps);
  // Graphs are keyed by the context bucket (kCtxBucket positions) holding
  // the pass's last row: the attention grid covers that bucket, so a replay
  // never launches more than one bucket's worth of idle partitions.
  const int bucket = (c->n + pos_off + M + kCtxBucket - 1) / kCtxBucket;
  std::string key;
  key.reserve(64 + c->cfg.n_layers);
  const intptr_t parts[9] = {M, pos_off, (intptr_t)tok, (intptr_t)arg, feats ? 1 : 0, bucket,
                             ps.save_row, ps.load ? 1 : 0, ps.head ? 1 : 0};
  key.append((const char*)parts, sizeof parts);
  if (skip) key.append((const char*)skip, c->cfg.n_layers);
  auto it = c->graphs.find(key);
  if (it == c->graphs.end()) {
    GraphEntry ge{};
    c->cap_part = std::min(c->lay.n_part, bucket * kCtxBucket / ATT_PT);
    HIPCHK(hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal));
    c->capturing = true;
    const ssd_status st = run_pass(c, tok, M, pos_off, skip, 0, M, arg, feats, ps);
    c->capturing = false;
    const hipError_t ee = hipStreamEndCapture(c->stream, &ge.graph);
    if (st != SSD_OK) {
      if (ee == hipSuccess) (void)hipGraphDestroy(ge.graph);
      return st;
    }
    HIPCHK(ee);
    const hipError_t ie = hipGraphInstantiate(&ge.exec, ge.graph, nullptr, nullptr, 0);
    if (ie != hipSuccess) {
      (void)hipGraphDestroy(ge.graph);
      return fail(SSD_E_HIP, "hipGraphInstantiate: %s", hipGetErrorString(ie));
    }
    it = c->graphs.emplace(key, ge).first;
  }
  HIPCHK(hipGraphLaunch(it->second.exec, c->stream));
  if (ps.head) c->head_rows = M;
  if (feats && c->cfg.n_feat > 0) c->feat_rows = M;
  return SSD_OK;
}

// Exit layer E of a tail mask (layers E..L-1 skipped, 1 <= E < L), else -1.
int tail_exit(const ssd_cfg& g, const uint8_t* mask) {
  if (!mask) return -1;
  int E = 0;
  while (E < g.n_layers && !mask[E]) ++E;
  if (E < 1 || E >= g.n_layers) return -1;
  for (int l = E; l < g.n_layers; ++l)
    if (!mask[l]) return -1;
  return E;
}

// Starts a draft with mask: remembers it and, with exit-state reuse on and a
// tail mask, its exit layer.
void set_kvq(ssd_ctx* c, const uint8_t* mask) {
  c->kvq_E = c->kvq_on ? tail_exit(c->cfg, mask) : -1;
  if (mask) c->kvq_mask.assign(mask, mask + c->cfg.n_layers);
  else c->kvq_mask.clear();
}

// Draft step j; with exit-state reuse on and a tail mask it also saves the
// row's state after the exit layer (LayerSkip summary 4.3.3: the exit query
// cache, read as the residual entering layer E).
ssd_status draft_step(ssd_ctx* c, int j, const uint8_t* mask) {
  PassSpec ps;
  if (c->kvq_E > 0) ps.save_row = j;
  return decode_pass(c, c->block + j, 1, j, mask, c->block + j + 1, false, ps);
}

// Verify of the drafted block [t_last, d_1..d_k].  With a saved exit state:
// d_k (the one row the draft did not run) goes through layers 0..E-1, then
// all k+1 rows run layers E..L-1 from the saved states; the KV entries of
// layers < E are the draft's.  Every row gets the arithmetic of the full
// pass (rows never depend on the pass width), so posterior and logits equal
// the full verify's bit for bit.
ssd_status verify_drafted(ssd_ctx* c, const uint8_t* mask, bool feats) {
  const int k = c->k;
  if (c->kvq_E > 0 && k > 0) {
    const int E = c->kvq_E, L = c->cfg.n_layers;
    PassSpec a;
    a.save_row = k;
    a.head = false;
    SSDCHK(decode_pass(c, c->block + k, 1, k, mask, nullptr, false, a));
    c->kvq_rest.assign(L, 0);
    for (int l = 0; l < E; ++l) c->kvq_rest[l] = 1;
    PassSpec b;
    b.load = true;
    return decode_pass(c, c->block, k + 1, 0, c->kvq_rest.data(), c->post, false, b);
  }
  return decode_pass(c, c->block, k + 1, 0, nullptr, c->post, feats);
}

ssd_status check_tokens(const ssd_cfg& g, const int32_t* t, int n) {
  for (int i = 0; i < n; ++i)
    if (t[i] < 0 || t[i] >= g.vocab) return fail(SSD_E_ARG, "token %d at index %d outside [0, %d)", t[i], i, g.vocab);
  return SSD_OK;
}

ssd_status transition(ssd_ctx* c, int op) {
  int next;
  SSDCHK(check_transition(c->state, op, &next));
  return SSD_OK;
}

void set_state(ssd_ctx* c, int op) {
  int next = c->state;
  check_transition(c->state, op, &next);
  c->state = next;
}

float elapsed(hipEvent_t a, hipEvent_t b) {
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return 0.f;
  return ms;
}

ssd_status do_prefill(ssd_ctx* c, const int32_t* tokens, int n) {
  const ssd_cfg& g = c->cfg;
  hipStream_t s = c->stream;
  const int P = g.prefill_chunk;
  c->n = 0;
  HIPCHK(launch_set_state(c->dstate, 0, 0, s));
  HIPCHK(launch_set_state(c->dstate, 1, 0, s));
  for (int s0 = 0; s0 < n; s0 += P) {
    const int rows = n - s0 < P ? n - s0 : P;
    HIPCHK(hipMemcpyAsync(c->toks, tokens + s0, rows * sizeof(int32_t), hipMemcpyHostToDevice, s));
    const bool last = s0 + rows == n;
    SSDCHK(run_pass(c, c->toks, rows, s0, nullptr, rows - 1, last ? 1 : 0, c->block, false));
  }
  HIPCHK(launch_set_state(c->dstate, 0, n, s));
  HIPCHK(launch_set_state(c->dstate, 1, 1, s));
  HIPCHK(launch_copy_tokens(c->block, c->outlog, 1, s));
  c->n = n;
  return SSD_OK;
}

ssd_status do_accept(ssd_ctx* c, bool sync, int* a_out, int* nemit_out) {
  hipStream_t s = c->stream;
  HIPCHK(launch_accept(c->block, c->post, c->k, c->dstate, c->outlog, c->result, s));
  if (sync) {
    HIPCHK(hipMemcpyAsync(c->hbuf, c->result, (c->k + 3) * sizeof(int), hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    if (a_out) *a_out = c->hbuf[0];
    if (nemit_out) *nemit_out = c->hbuf[1];
  }
  return SSD_OK;
}

// Copies every bf16 GEMM weight into the packed tile layout in the workspace
// (see device.h) and points the context at the copies; the caller's buffers
// of these matrices are not read after this.
hipError_t pack_weights(ssd_ctx* c) {
  const ssd_cfg& g = c->cfg;
  const int d = g.d_model, hq = g.n_q_heads, hkv = g.n_kv_heads, hd = g.head_dim;
  uint16_t* wp = (uint16_t*)at(c, c->lay.wpack);
  size_t off = 0;
  hipError_t e = hipSuccess;
  auto pack = [&](const void* s0, const void* s1, const void* s2, int N, int K, int mode, int pair, int tw = 16) {
    uint16_t* dst = wp + off;
    off += (size_t)N * K * (pair ? 2 : 1);
    if (e == hipSuccess) {
      PackArgs p{};
      p.src0 = s0; p.src1 = s1; p.src2 = s2; p.dst = dst; p.N = N; p.K = K; p.mode = mode; p.pair = pair; p.tw = tw;
      p.hq = hq; p.hkv = hkv; p.hd = hd;
      e = launch_pack(p, c->stream);
    }
    return (const void*)dst;
  };
  auto el = [](const void* p, size_t i) { return (const void*)((const uint16_t*)p + i); };
  for (LayerW& w : c->L) {
    w.wq = pack(w.wq, w.wk, w.wv, (hq + 2 * hkv) * hd, d, 1, 0, qkv_tile_width(hq, hkv, hd));
    w.wk = w.wv = nullptr;
    w.wo = pack(w.wo, nullptr, nullptr, d, hq * hd, 0, 0, resid_tile_width(d));   // as launch_gemm reads it
    if (w.moe) {
      const int E = g.n_experts, fe = g.expert_ffn, S = g.n_shared;
      w.router = pack(w.router, nullptr, nullptr, E, d, 0, 0);
      const void* eg = nullptr;
      for (int x = 0; x < E; ++x) {
        const void* p = pack(el(w.eg, (size_t)x * fe * d), el(w.eu, (size_t)x * fe * d), nullptr, fe, d, 0, 1);
        if (!x) eg = p;
      }
      const void* ed = nullptr;
      for (int x = 0; x < E; ++x) {
        const void* p = pack(el(w.ed, (size_t)x * d * fe), nullptr, nullptr, d, fe, 0, 0);
        if (!x) ed = p;
      }
      const void* sg = nullptr;
      for (int x = 0; x < S; ++x) {
        const void* p = pack(el(w.sg, (size_t)x * fe * d), el(w.su, (size_t)x * fe * d), nullptr, fe, d, 0, 1);
        if (!x) sg = p;
      }
      const void* sd = nullptr;
      for (int x = 0; x < S; ++x) {
        const void* p = pack(el(w.sd, (size_t)x * d * fe), nullptr, nullptr, d, fe, 0, 0);
        if (!x) sd = p;
      }
      w.eg = eg; w.ed = ed; w.sg = sg; w.sd = sd;
      w.eu = w.su = nullptr;
    } else {
      w.w_gate = pack(w.w_gate, w.w_up, nullptr, w.ffn, d, 0, 1, swiglu_tile_width(w.ffn));   // as launch_gemm reads it
      w.w_up = nullptr;
      w.w_down = pack(w.w_down, nullptr, nullptr, d, w.ffn, 0, 0, resid_tile_width(d));
    }
  }
  c->lm_head = pack(c->lm_head, nullptr, nullptr, g.vocab, d, 0, 0);
  if (c->fc) c->fc = pack(c->fc, nullptr, nullptr, d, g.n_feat * d, 0, 0);
  if (e != hipSuccess) return e;
  if ((int64_t)off != packed_elems(g)) return hipErrorInvalidValue;   // layout and packing disagree
  return hipStreamSynchronize(c->stream);
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

ssd_status ssd_load(const ssd_cfg* cfg, const ssd_buf* weights, int32_t n_weights, ssd_buf workspace,
                    void* hip_stream, ssd_ctx** out) {
  clear_error();
  if (!out) return fail(SSD_E_ARG, "out is NULL");
  *out = nullptr;
  SSDCHK(validate(cfg));
  Layout lay;
  compute_layout(*cfg, lay);
  auto table = weight_table(*cfg);
  if (!weights || n_weights != (int32_t)table.size())
    return fail(SSD_E_ARG, "expected %d weight buffers, got %d", (int)table.size(), n_weights);
  const size_t esz = cfg->dtype == SSD_BF16 ? 2 : 4;
  for (int i = 0; i < n_weights; ++i) {
    if (!weights[i].ptr && table[i] != 0) return fail(SSD_E_ARG, "weight %d is NULL", i);
    if (weights[i].nbytes != (int64_t)(table[i] * esz))
      return fail(SSD_E_ARG, "weight %d has %lld bytes, expected %lld", i, (long long)weights[i].nbytes,
                  (long long)(table[i] * esz));
    if ((uintptr_t)weights[i].ptr % 16) return fail(SSD_E_ARG, "weight %d is not 16-byte aligned", i);
  }
  if (!workspace.ptr || workspace.nbytes < (int64_t)lay.total)
    return fail(SSD_E_ARG, "workspace needs %lld bytes", (long long)lay.total);
  if ((uintptr_t)workspace.ptr % 256) return fail(SSD_E_ARG, "workspace is not 256-byte aligned");

  ssd_ctx* c = new ssd_ctx();
  c->cfg = *cfg;
  c->lay = lay;
  c->stream = (hipStream_t)hip_stream;
  c->ws = (char*)workspace.ptr;
  c->esz = esz;
  int wi = 0;
  c->embed = weights[wi++].ptr;
  for (int l = 0; l < cfg->n_layers; ++l) {
    LayerW w{};
    w.attn_norm = weights[wi++].ptr;
    w.wq = weights[wi++].ptr;
    w.wk = weights[wi++].ptr;
    w.wv = weights[wi++].ptr;
    w.wo = weights[wi++].ptr;
    w.ffn_norm = weights[wi++].ptr;
    w.moe = is_moe_layer(*cfg, l);
    if (w.moe) {
      w.router = weights[wi++].ptr;
      w.eg = weights[wi++].ptr;
      w.eu = weights[wi++].ptr;
      w.ed = weights[wi++].ptr;
      w.sg = weights[wi++].ptr;
      w.su = weights[wi++].ptr;
      w.sd = weights[wi++].ptr;
    } else {
      w.w_gate = weights[wi++].ptr;
      w.w_up = weights[wi++].ptr;
      w.w_down = weights[wi++].ptr;
      w.ffn = layer_ffn(*cfg);
    }
    w.feat_slot = -1;
    for (int i = 0; i < cfg->n_feat; ++i)
      if (cfg->feat_layers[i] == l) w.feat_slot = i;
    c->L.push_back(w);
  }
  c->final_norm = weights[wi++].ptr;
  c->lm_head = weights[wi++].ptr;
  c->fc = cfg->n_feat > 0 ? weights[wi++].ptr : nullptr;

  c->kc = at(c, lay.kc); c->vc = at(c, lay.vc);
  c->x = (float*)at(c, lay.x); c->ss = (float*)at(c, lay.ss); c->xn = at(c, lay.xn); c->q = at(c, lay.q); c->att = at(c, lay.att);
  c->act = at(c, lay.act); c->logits = (float*)at(c, lay.logits);
  c->amax_v = (float*)at(c, lay.amax_v); c->amax_i = (int*)at(c, lay.amax_i);
  c->trace = (float*)at(c, lay.trace);
  c->trace_pts = (char*)at(c, lay.trace_pts);
  c->tp = trace_points(*cfg);
  c->exit_x = (float*)at(c, lay.exit_x);
  c->exit_ss = (float*)at(c, lay.exit_ss);
  c->dlog = (float*)at(c, lay.dlog);
  c->tout = (int*)at(c, lay.tout);
  c->smp = SmpBufs{at(c, lay.smp_stats), (float*)at(c, lay.smp_csum), at(c, lay.smp_ctl), (int)lay.smp_nch};
  c->part_o = (float*)at(c, lay.part_o); c->part_ml = (float*)at(c, lay.part_ml);
  c->cos_t = (float*)at(c, lay.rope_cos); c->sin_t = (float*)at(c, lay.rope_sin);
  c->block = (int*)at(c, lay.block); c->post = (int*)at(c, lay.post); c->toks = (int*)at(c, lay.toks);
  c->dstate = (int*)at(c, lay.state); c->result = (int*)at(c, lay.result); c->outlog = (int*)at(c, lay.outlog);
  c->tblock = (int*)at(c, lay.tblock); c->tpost = (int*)at(c, lay.tpost); c->tstate = (int*)at(c, lay.tstate);
  c->tresult = (int*)at(c, lay.tresult); c->toutlog = (int*)at(c, lay.toutlog);
  c->tap = cfg->n_feat ? at(c, lay.tap) : nullptr;
  c->feat = cfg->n_feat ? at(c, lay.feat) : nullptr;
  if (lay.frag) {
    c->xn_p = at(c, lay.xn_p); c->att_p = at(c, lay.att_p); c->act_p = at(c, lay.act_p);
    c->tap_p = cfg->n_feat ? at(c, lay.tap_p) : nullptr;
  }
  if (cfg->n_experts > 0) {
    c->m_rlogits = (float*)at(c, lay.m_rlogits); c->m_ids = (int*)at(c, lay.m_ids);
    c->m_gates = (float*)at(c, lay.m_gates); c->m_inject = (int*)at(c, lay.m_inject);
    c->m_slot_out = (float*)at(c, lay.m_slot_out); c->m_groups = (int*)at(c, lay.m_groups);
    c->m_union = (int*)at(c, lay.m_union);
    c->m_rstd = (float*)at(c, lay.m_rstd);
  }

  ssd_status st = SSD_OK;
  auto cleanup = [&](ssd_status s) { ssd_free(c); return s; };
  // rotary tables, computed in double on the host: angle = pos * theta^(-2i/hd)
  {
    const int half = cfg->head_dim / 2;
    std::vector<float> cs((size_t)cfg->max_ctx * half), sn((size_t)cfg->max_ctx * half);
    for (int p = 0; p < cfg->max_ctx; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * std::pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
        cs[(size_t)p * half + i] = (float)std::cos(ang);
        sn[(size_t)p * half + i] = (float)std::sin(ang);
      }
    hipError_t e = hipMemsetAsync(c->ws, 0, lay.total, c->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(c->cos_t, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(c->sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e == hipSuccess) e = hipHostMalloc((void**)&c->hbuf, 4096, hipHostMallocDefault);
    for (int i = 0; i < EV_N && e == hipSuccess; ++i) e = hipEventCreate(&c->ev[i]);
    if (e != hipSuccess) {
      st = fail(SSD_E_HIP, "load: %s", hipGetErrorString(e));
      return cleanup(st);
    }
  }
  if (cfg->dtype == SSD_BF16) {
    const hipError_t e = pack_weights(c);
    if (e != hipSuccess) {
      st = fail(SSD_E_HIP, "load (weight packing): %s", hipGetErrorString(e));
      return cleanup(st);
    }
  }
  memset(&c->st, 0, sizeof c->st);
  *out = c;
  return SSD_OK;
}

void ssd_free(ssd_ctx* c) {
  if (!c) return;
  (void)hipStreamSynchronize(c->stream);
  destroy_graphs(c);
  for (int i = 0; i < EV_N; ++i)
    if (c->ev[i]) (void)hipEventDestroy(c->ev[i]);
  if (c->hbuf) (void)hipHostFree(c->hbuf);
  delete c;
}

ssd_status ssd_reset(ssd_ctx* c) {
  clear_error();
  if (!c) return fail(SSD_E_ARG, "ctx is NULL");
  SSDCHK(transition(c, SSD_OP_RESET));
  HIPCHK(launch_set_state(c->dstate, 0, 0, c->stream));
  HIPCHK(launch_set_state(c->dstate, 1, 0, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  c->n = 0;
  c->k = 0;
  c->kvq_E = -1;
  memset(&c->st, 0, sizeof c->st);
  set_state(c, SSD_OP_RESET);
  return SSD_OK;
}

int32_t ssd_state(const ssd_ctx* c) { return c ? c->state : -1; }
int32_t ssd_context_length(const ssd_ctx* c) { return c ? c->n : -1; }

ssd_status ssd_prefill(ssd_ctx* c, const int32_t* tokens, int32_t n, int32_t* next_tok) {
  clear_error();
  if (!c || !tokens) return fail(SSD_E_ARG, "NULL argument");
  SSDCHK(transition(c, SSD_OP_PREFILL));
  if (n < 1) return fail(SSD_E_ARG, "empty prompt");
  if (n + 1 > c->cfg.max_ctx) return fail(SSD_E_CAPACITY, "prompt of %d tokens needs max_ctx > %d", n, n);
  SSDCHK(check_tokens(c->cfg, tokens, n));
  auto t0 = std::chrono::steady_clock::now();
  SSDCHK(do_prefill(c, tokens, n));
  if (next_tok) HIPCHK(hipMemcpyAsync(c->hbuf, c->block, 4, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  if (next_tok) *next_tok = c->hbuf[0];
  c->st.t_prefill_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  set_state(c, SSD_OP_PREFILL);
  return SSD_OK;
}

ssd_status ssd_draft(ssd_ctx* c, const uint8_t* skip_mask, int32_t k, int32_t* drafts) {
  clear_error();
  if (!c) return fail(SSD_E_ARG, "ctx is NULL");
  SSDCHK(transition(c, SSD_OP_DRAFT));
  if (k < 1 || k + 1 > c->cfg.max_block) return fail(SSD_E_ARG, "k=%d outside [1, max_block-1=%d]", k, c->cfg.max_block - 1);
  if (c->n + k + 1 > c->cfg.max_ctx) return fail(SSD_E_CAPACITY, "n=%d + k+1=%d exceeds max_ctx=%d", c->n, k + 1, c->cfg.max_ctx);
  set_kvq(c, skip_mask);
  HIPCHK(hipEventRecord(c->ev[EV_A], c->stream));
  for (int j = 0; j < k; ++j) SSDCHK(draft_step(c, j, skip_mask));
  HIPCHK(hipEventRecord(c->ev[EV_B], c->stream));
  c->k = k;
  if (drafts) HIPCHK(hipMemcpyAsync(c->hbuf, c->block + 1, k * sizeof(int), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  if (drafts) memcpy(drafts, c->hbuf, k * sizeof(int));
  c->st.t_draft_ms += elapsed(c->ev[EV_A], c->ev[EV_B]);
  c->st.drafted += k;
  set_state(c, SSD_OP_DRAFT);
  return SSD_OK;
}

ssd_status ssd_verify(ssd_ctx* c, const int32_t* block, int32_t m, int32_t* posterior) {
  clear_error();
  if (!c) return fail(SSD_E_ARG, "ctx is NULL");
  const int op = block ? SSD_OP_VERIFY_BLOCK : SSD_OP_VERIFY;
  SSDCHK(transition(c, op));
  if (block) {
    if (m < 1 || m > c->cfg.max_block) return fail(SSD_E_ARG, "m=%d outside [1, max_block=%d]", m, c->cfg.max_block);
    SSDCHK(check_tokens(c->cfg, block, m));
  } else if (m != c->k + 1) {
    return fail(SSD_E_ARG, "m=%d but the drafted block has %d tokens", m, c->k + 1);
  }
  if (c->n + m + 1 > c->cfg.max_ctx) return fail(SSD_E_CAPACITY, "n=%d + m=%d exceeds max_ctx=%d", c->n, m, c->cfg.max_ctx);
  if (block) {
    memcpy(c->hbuf, block, m * sizeof(int));
    HIPCHK(hipMemcpyAsync(c->block, c->hbuf, m * sizeof(int), hipMemcpyHostToDevice, c->stream));
    c->k = m - 1;
    c->kvq_E = -1;   // the saved exit states belong to the drafted tokens, not to this block
  }
  HIPCHK(hipEventRecord(c->ev[EV_A], c->stream));
  SSDCHK(verify_drafted(c, c->kvq_mask.empty() ? nullptr : c->kvq_mask.data(), true));
  c->kvq_E = -1;
  HIPCHK(hipEventRecord(c->ev[EV_B], c->stream));
  HIPCHK(hipMemcpyAsync(c->hbuf, c->post, m * sizeof(int), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  if (posterior) memcpy(posterior, c->hbuf, m * sizeof(int));
  c->st.t_verify_ms += elapsed(c->ev[EV_A], c->ev[EV_B]);
  c->st.verify_passes += 1;
  set_state(c, op);
  return SSD_OK;
}

ssd_status ssd_accept_rollback(ssd_ctx* c, int32_t* n_accepted, int32_t* emitted, int32_t* n_emitted) {
  clear_error();
  if (!c) return fail(SSD_E_ARG, "ctx is NULL");
  SSDCHK(transition(c, SSD_OP_ACCEPT));
  int a = 0, ne = 0;
  SSDCHK(do_accept(c, true, &a, &ne));
  if (n_accepted) *n_accepted = a;
  if (n_emitted) *n_emitted = ne;
  if (emitted) memcpy(emitted, c->hbuf + 2, ne * sizeof(int));
  c->n += ne;
  c->st.cycles += 1;
  c->st.accepted += a;
  c->st.emitted += ne;
  set_state(c, SSD_OP_ACCEPT);
  return SSD_OK;
}

ssd_status ssd_generate(ssd_ctx* c, const int32_t* prompt, int32_t n_prompt, int32_t n_new, int32_t greedy,
                        const uint8_t* skip_mask, int32_t k, int32_t* out, ssd_stats* stats) {
  clear_error();
  if (!c || !prompt || !out) return fail(SSD_E_ARG, "NULL argument");
  if (greedy != 0 && greedy != 1) return fail(SSD_E_UNSUPPORTED, "greedy must be 1 (greedy) or 0 (sampling)");
  const bool sampled = greedy == 0;
  if (sampled && !c->smp_set) return fail(SSD_E_STATE, "sampling parameters not set (ssd_set_sampling)");
  if (n_prompt < 1 || n_new < 1) return fail(SSD_E_ARG, "n_prompt and n_new must be positive");
  const bool spec = skip_mask != nullptr && k > 0;
  if (spec && k + 1 > c->cfg.max_block) return fail(SSD_E_ARG, "k=%d exceeds max_block-1", k);
  if (k < 0) return fail(SSD_E_ARG, "negative k");
  const int kk = spec ? k : 0;
  if (n_prompt + n_new + kk + 1 > c->cfg.max_ctx)
    return fail(SSD_E_CAPACITY, "prompt %d + %d new + block %d exceeds max_ctx %d", n_prompt, n_new, kk + 1, c->cfg.max_ctx);
  SSDCHK(check_tokens(c->cfg, prompt, n_prompt));
  if (c->state != SSD_ST_LOADED) SSDCHK(ssd_reset(c));
  memset(&c->st, 0, sizeof c->st);
  SSDCHK(ssd_prefill(c, prompt, n_prompt, nullptr));
  hipStream_t s = c->stream;
  const int V = c->cfg.vocab;
  if (sampled)
    HIPCHK(launch_first_sample(c->logits, V, c->smp_T, c->smp_seed, c->block, c->dstate, c->outlog, c->smp, s));
  auto t0 = std::chrono::steady_clock::now();
  int produced = 1;
  if (!spec) {
    // plain greedy: one full pass per token, positions and tokens device-resident
    c->k = 0;
    HIPCHK(hipEventRecord(c->ev[EV_A], s));
    for (int i = 1; i < n_new; ++i) {
      SSDCHK(decode_pass(c, c->block, 1, 0, nullptr, c->post, false));
      if (sampled)   // the k = 0 cycle: one token drawn from p_0
        HIPCHK(launch_spec_accept(c->logits, c->dlog, V, V, 0, c->smp_T, c->smp_seed, c->block, c->dstate, c->outlog,
                                  c->result, nullptr, c->smp, s));
      else
        SSDCHK(do_accept(c, false, nullptr, nullptr));
      c->n += 1;
    }
    HIPCHK(hipEventRecord(c->ev[EV_B], s));
    HIPCHK(hipStreamSynchronize(s));
    produced = n_new;
    c->st.cycles = n_new - 1;
    c->st.emitted = n_new - 1;
    c->st.verify_passes = n_new - 1;
    c->st.t_verify_ms = elapsed(c->ev[EV_A], c->ev[EV_B]);
  } else {
    while (produced < n_new) {
      HIPCHK(hipEventRecord(c->ev[EV_A], s));
      if (sampled) c->kvq_E = -1;
      else set_kvq(c, skip_mask);
      for (int j = 0; j < k; ++j) {
        SSDCHK(draft_step(c, j, skip_mask));
        if (sampled)   // d_{j+1} ~ q_{j+1}; the draft row is kept for the accept
          HIPCHK(launch_draft_sample(c->logits, V, c->smp_T, c->smp_seed, c->block, c->dstate, j,
                                     c->dlog + (size_t)j * V, c->smp, s));
      }
      c->k = k;
      HIPCHK(hipEventRecord(c->ev[EV_B], s));
      SSDCHK(verify_drafted(c, skip_mask, true));
      c->kvq_E = -1;
      HIPCHK(hipEventRecord(c->ev[EV_C], s));
      int a = 0, ne = 0;
      if (sampled)
        HIPCHK(launch_spec_accept(c->logits, c->dlog, V, V, k, c->smp_T, c->smp_seed, c->block, c->dstate, c->outlog,
                                  c->result, nullptr, c->smp, s));
      else
        HIPCHK(launch_accept(c->block, c->post, k, c->dstate, c->outlog, c->result, s));
      HIPCHK(hipEventRecord(c->ev[EV_D], s));
      HIPCHK(hipMemcpyAsync(c->hbuf, c->result, 2 * sizeof(int), hipMemcpyDeviceToHost, s));
      HIPCHK(hipStreamSynchronize(s));
      a = c->hbuf[0];
      ne = c->hbuf[1];
      c->n += ne;
      produced += ne;
      c->st.cycles += 1;
      c->st.drafted += k;
      c->st.accepted += a;
      c->st.emitted += ne;
      c->st.verify_passes += 1;
      c->st.t_draft_ms += elapsed(c->ev[EV_A], c->ev[EV_B]);
      c->st.t_verify_ms += elapsed(c->ev[EV_B], c->ev[EV_C]);
      c->st.t_accept_ms += elapsed(c->ev[EV_C], c->ev[EV_D]);
    }
  }
  std::vector<int32_t> tmp(n_new);
  HIPCHK(hipMemcpyAsync(tmp.data(), c->outlog, n_new * sizeof(int32_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  c->st.t_decode_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  memcpy(out, tmp.data(), n_new * sizeof(int32_t));
  c->state = SSD_ST_READY;
  if (stats) *stats = c->st;
  return SSD_OK;
}

ssd_status ssd_set_option(ssd_ctx* c, int32_t option, int32_t value) {
  clear_error();
  if (!c) return fail(SSD_E_ARG, "ctx is NULL");
  if (option != SSD_OPT_GRAPHS && option != SSD_OPT_MOE_DEDUP && option != SSD_OPT_TRACE && option != SSD_OPT_KVQ &&
      option != SSD_OPT_TILE_GROUPS)
    return fail(SSD_E_ARG, "unknown option %d", option);
  if (option == SSD_OPT_TILE_GROUPS && value < 0) return fail(SSD_E_ARG, "tile groups threshold must be >= 0");
  if (option == SSD_OPT_MOE_DEDUP && c->cfg.n_experts == 0) return fail(SSD_E_UNSUPPORTED, "not an MoE model");
  HIPCHK(hipStreamSynchronize(c->stream));
  destroy_graphs(c);
  if (option == SSD_OPT_GRAPHS) c->use_graphs = value != 0;
  else if (option == SSD_OPT_TRACE) c->trace_on = value != 0;
  else if (option == SSD_OPT_KVQ) c->kvq_on = value != 0;
  else if (option == SSD_OPT_TILE_GROUPS) c->tile_wg_min = value;
  else c->cfg.moe_dedup = value != 0;
  return SSD_OK;
}

ssd_status ssd_set_sampling(ssd_ctx* c, float temperature, uint64_t seed) {
  clear_error();
  if (!c) return fail(SSD_E_ARG, "ctx is NULL");
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return fail(SSD_E_ARG, "temperature must be > 0 and finite");
  c->smp_set = true;
  c->smp_T = temperature;
  c->smp_seed = seed;
  return SSD_OK;
}

ssd_status ssd_test_spec_cycle(ssd_ctx* c, const float* target, const float* draft, int32_t k, int32_t V,
                               float temperature, uint64_t seed, uint64_t cycle0, int32_t trials, int32_t* out) {
  clear_error();
  if (!c || !target || !out || (k > 0 && !draft)) return fail(SSD_E_ARG, "NULL argument");
  if (k < 0 || k + 1 > c->cfg.max_block) return fail(SSD_E_ARG, "k=%d outside [0, max_block-1]", k);
  if (V < 1 || V > c->cfg.vocab) return fail(SSD_E_ARG, "V=%d outside [1, vocab]", V);
  if (trials < 1) return fail(SSD_E_ARG, "trials < 1");
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return fail(SSD_E_ARG, "temperature must be > 0 and finite");
  hipStream_t s = c->stream;
  HIPCHK(hipMemcpyAsync(c->logits, target, (size_t)(k + 1) * V * 4, hipMemcpyHostToDevice, s));
  if (k > 0) HIPCHK(hipMemcpyAsync(c->dlog, draft, (size_t)k * V * 4, hipMemcpyHostToDevice, s));
  // the decode loop's kernels, one cycle after another on the test state:
  // cycle counter tstate[2] from cycle0, drafts into tblock[1..k]
  int st[16] = {0};
  if (cycle0 + (uint64_t)trials > (uint64_t)INT32_MAX) return fail(SSD_E_ARG, "cycle0 + trials exceeds 2^31 - 1");
  st[2] = (int)cycle0;
  HIPCHK(hipMemcpyAsync(c->tstate, st, sizeof st, hipMemcpyHostToDevice, s));
  for (int t0 = 0; t0 < trials; t0 += kTestCycles) {
    const int n = std::min(kTestCycles, trials - t0);
    for (int t = 0; t < n; ++t) {
      for (int j = 0; j < k; ++j)
        HIPCHK(launch_draft_sample(c->dlog + (size_t)j * V, V, temperature, seed, c->tblock, c->tstate, j, nullptr,
                                   c->smp, s));
      HIPCHK(launch_spec_accept(c->logits, c->dlog, V, V, k, temperature, seed, c->tblock, c->tstate, nullptr,
                                c->tresult, c->tout + (size_t)t * (k + 2), c->smp, s));
    }
    HIPCHK(hipMemcpyAsync(out + (size_t)t0 * (k + 2), c->tout, (size_t)n * (k + 2) * 4, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
  }
  c->head_rows = 0;
  return SSD_OK;
}

ssd_status ssd_get_stats(const ssd_ctx* c, ssd_stats* stats) {
  if (!c || !stats) return fail(SSD_E_ARG, "NULL argument");
  *stats = c->st;
  return SSD_OK;
}

ssd_status ssd_read_logits(ssd_ctx* c, float* host, int32_t rows) {
  clear_error();
  if (!c || !host) return fail(SSD_E_ARG, "NULL argument");
  if (rows < 1 || rows > c->head_rows) return fail(SSD_E_ARG, "rows=%d but the last pass has %d", rows, c->head_rows);
  HIPCHK(hipMemcpyAsync(host, c->logits, (size_t)rows * c->cfg.vocab * 4, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  return SSD_OK;
}

ssd_status ssd_read_trace(ssd_ctx* c, float* host, int32_t rows) {
  clear_error();
  if (!c || !host) return fail(SSD_E_ARG, "NULL argument");
  if (!c->trace_on) return fail(SSD_E_STATE, "residual trace is off (SSD_OPT_TRACE)");
  if (rows < 1 || rows > c->head_rows || rows > c->cfg.max_block)
    return fail(SSD_E_ARG, "rows=%d but the last pass has %d", rows, c->head_rows);
  const size_t d = c->cfg.d_model;
  for (int l = 0; l < c->cfg.n_layers; ++l)
    HIPCHK(hipMemcpyAsync(host + (size_t)l * rows * d, c->trace + (size_t)l * c->cfg.max_block * d,
                          rows * d * 4, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  return SSD_OK;
}

ssd_status ssd_read_trace_point(ssd_ctx* c, int32_t layer, int32_t point, int32_t rows, void* host) {
  clear_error();
  if (!c || !host) return fail(SSD_E_ARG, "NULL argument");
  if (!c->trace_on) return fail(SSD_E_STATE, "residual trace is off (SSD_OPT_TRACE)");
  const ssd_cfg& g = c->cfg;
  if (layer < 0 || layer > g.n_layers || point < 0 || point > 5 || (layer == g.n_layers && point != 0))
    return fail(SSD_E_ARG, "no trace point %d of layer %d", point, layer);
  if (rows < 1 || rows > c->last_M || rows > g.max_block)
    return fail(SSD_E_ARG, "rows=%d but the last pass has %d", rows, c->last_M);
  const size_t off = (size_t)layer * c->tp.layer + (layer < g.n_layers ? c->tp.off[point] : 0);
  size_t row = layer < g.n_layers ? c->tp.row[point] : c->tp.row[0];
  if (layer < g.n_layers && point == 5)   // the layer's own activation width
    row = (c->L[layer].moe ? (size_t)(g.top_k + g.n_shared) * g.expert_ffn : (size_t)c->L[layer].ffn) * c->esz;
  HIPCHK(hipMemcpyAsync(host, c->trace_pts + off, rows * row, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  return SSD_OK;
}

ssd_status ssd_layer_cosines(ssd_ctx* c, int32_t rows, double* cos) {
  clear_error();
  if (!c || !cos) return fail(SSD_E_ARG, "NULL argument");
  if (!c->trace_on) return fail(SSD_E_STATE, "residual trace is off (SSD_OPT_TRACE)");
  if (!c->last_tok || !c->last_full) return fail(SSD_E_STATE, "the last decode-loop pass did not run every layer");
  if (rows < 1 || rows > c->last_M || rows > c->cfg.max_block)
    return fail(SSD_E_ARG, "rows=%d but the last pass has %d", rows, c->last_M);
  const ssd_cfg& g = c->cfg;
  const size_t d = g.d_model, L = g.n_layers;
  std::vector<int> tok(rows);
  std::vector<float> tr(L * rows * d), in((size_t)rows * d);
  std::vector<char> emb((size_t)rows * d * c->esz);
  HIPCHK(hipMemcpyAsync(tok.data(), c->last_tok, rows * sizeof(int), hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  for (int r = 0; r < rows; ++r) {
    if (tok[r] < 0 || tok[r] >= g.vocab) return fail(SSD_E_HIP, "token buffer holds %d", tok[r]);
    HIPCHK(hipMemcpyAsync(emb.data() + (size_t)r * d * c->esz, (const char*)c->embed + (size_t)tok[r] * d * c->esz,
                          d * c->esz, hipMemcpyDeviceToHost, c->stream));
  }
  for (size_t l = 0; l < L; ++l)
    HIPCHK(hipMemcpyAsync(tr.data() + l * rows * d, c->trace + l * g.max_block * d, rows * d * 4,
                          hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  for (size_t i = 0; i < (size_t)rows * d; ++i) {
    if (c->esz == 2) {
      uint32_t u = (uint32_t)((const uint16_t*)emb.data())[i] << 16;
      float f;
      memcpy(&f, &u, 4);
      in[i] = f;
    } else {
      in[i] = ((const float*)emb.data())[i];
    }
  }
  for (size_t l = 0; l < L; ++l) {
    const float* a = l == 0 ? in.data() : tr.data() + (l - 1) * rows * d;
    const float* b = tr.data() + l * rows * d;
    double sum = 0.0;
    for (int r = 0; r < rows; ++r) {
      double ab = 0.0, aa = 0.0, bb = 0.0;
      for (size_t i = 0; i < d; ++i) {
        const double x = a[(size_t)r * d + i], y = b[(size_t)r * d + i];
        ab += x * y;
        aa += x * x;
        bb += y * y;
      }
      sum += ab / std::sqrt(aa * bb);
    }
    cos[l] = sum / rows;
  }
  return SSD_OK;
}

ssd_status ssd_read_kv(ssd_ctx* c, int32_t layer, int32_t pos0, int32_t n, void* k_host, void* v_host) {
  clear_error();
  if (!c || !k_host || !v_host) return fail(SSD_E_ARG, "NULL argument");
  const ssd_cfg& g = c->cfg;
  if (layer < 0 || layer >= g.n_layers || pos0 < 0 || n < 1 || pos0 + n > g.max_ctx)
    return fail(SSD_E_ARG, "layer/positions out of range");
  const size_t hd = g.head_dim, row = hd * c->esz, ld = kv_stride(g), esz = c->esz;
  // V rows are head dims ([dim][position]): gather [h][dim][n] then transpose
  std::vector<char> vt((size_t)g.n_kv_heads * hd * n * esz);
  for (int h = 0; h < g.n_kv_heads; ++h) {
    const size_t koff = (((size_t)layer * g.n_kv_heads + h) * ld + pos0) * row;
    HIPCHK(hipMemcpyAsync((char*)k_host + (size_t)h * n * row, (char*)c->kc + koff, n * row, hipMemcpyDeviceToHost, c->stream));
    const size_t voff = (((size_t)layer * g.n_kv_heads + h) * hd * ld + pos0) * esz;
    HIPCHK(hipMemcpy2DAsync(vt.data() + (size_t)h * hd * n * esz, n * esz, (char*)c->vc + voff, ld * esz, n * esz, hd,
                            hipMemcpyDeviceToHost, c->stream));
  }
  HIPCHK(hipStreamSynchronize(c->stream));
  for (int h = 0; h < g.n_kv_heads; ++h)
    for (size_t dd = 0; dd < hd; ++dd)
      for (int r = 0; r < n; ++r)
        memcpy((char*)v_host + (((size_t)h * n + r) * hd + dd) * esz, vt.data() + (((size_t)h * hd + dd) * n + r) * esz, esz);
  return SSD_OK;
}

ssd_status ssd_read_features(ssd_ctx* c, uint16_t* host, int32_t rows) {
  clear_error();
  if (!c || !host) return fail(SSD_E_ARG, "NULL argument");
  if (c->cfg.n_feat == 0) return fail(SSD_E_UNSUPPORTED, "no feature tap configured");
  if (c->cfg.dtype != SSD_BF16) return fail(SSD_E_UNSUPPORTED, "features are read as bf16");
  if (rows < 1 || rows > c->feat_rows) return fail(SSD_E_ARG, "rows=%d but the last verify had %d", rows, c->feat_rows);
  HIPCHK(hipMemcpyAsync(host, c->feat, (size_t)rows * c->cfg.d_model * 2, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  return SSD_OK;
}

ssd_status ssd_set_routing(ssd_ctx* c, const int32_t* ids, int32_t n) {
  clear_error();
  if (!c) return fail(SSD_E_ARG, "ctx is NULL");
  if (c->cfg.n_experts == 0) return fail(SSD_E_UNSUPPORTED, "not an MoE model");
  if (n != 0 && (!ids || n < 0 || n > c->lay.R)) return fail(SSD_E_ARG, "n=%d outside [0, %d]", n, c->lay.R);
  // Captured passes bake in where the expert ids come from (the router's
  // choice or the injected buffer): switching between the two drops them.
  // The injected ids themselves are read from device memory at replay.
  if ((n == 0) != (c->moe_inject == 0)) {
    HIPCHK(hipStreamSynchronize(c->stream));
    destroy_graphs(c);
  }
  if (n == 0) { c->moe_inject = 0; return SSD_OK; }
  const ssd_cfg& g = c->cfg;
  std::vector<int32_t> buf((size_t)g.n_layers * c->lay.R * g.top_k, 0);
  for (int l = 0; l < g.n_layers; ++l)
    for (int t = 0; t < n; ++t)
      for (int j = 0; j < g.top_k; ++j) {
        const int32_t e = ids[((size_t)l * n + t) * g.top_k + j];
        if (is_moe_layer(g, l) && (e < 0 || e >= g.n_experts)) return fail(SSD_E_ARG, "expert id %d out of range", e);
        buf[((size_t)l * c->lay.R + t) * g.top_k + j] = is_moe_layer(g, l) ? e : 0;
      }
  HIPCHK(hipMemcpyAsync(c->m_inject, buf.data(), buf.size() * 4, hipMemcpyHostToDevice, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  c->moe_inject = n;
  return SSD_OK;
}

ssd_status ssd_read_union(ssd_ctx* c, int32_t* host) {
  clear_error();
  if (!c || !host) return fail(SSD_E_ARG, "NULL argument");
  if (c->cfg.n_experts == 0) return fail(SSD_E_UNSUPPORTED, "not an MoE model");
  HIPCHK(hipMemcpyAsync(host, c->m_union, c->cfg.n_layers * 4, hipMemcpyDeviceToHost, c->stream));
  HIPCHK(hipStreamSynchronize(c->stream));
  return SSD_OK;
}

ssd_status ssd_test_accept(ssd_ctx* c, const int32_t* d, const int32_t* p, int32_t k, int32_t* a) {
  clear_error();
  if (!c || !p || !a || (k > 0 && !d)) return fail(SSD_E_ARG, "NULL argument");
  if (k < 0 || k + 1 > SSD_MAX_BLOCK) return fail(SSD_E_ARG, "k=%d outside [0, %d]", k, SSD_MAX_BLOCK - 1);
  int* h = c->hbuf;
  h[0] = -1;
  for (int i = 0; i < k; ++i) h[1 + i] = d[i];
  for (int i = 0; i <= k; ++i) h[64 + i] = p[i];
  for (int i = 0; i < 16; ++i) h[128 + i] = 0;
  hipStream_t s = c->stream;
  HIPCHK(hipMemcpyAsync(c->tblock, h, (k + 1) * 4, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(c->tpost, h + 64, (k + 1) * 4, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemcpyAsync(c->tstate, h + 128, 16 * 4, hipMemcpyHostToDevice, s));
  HIPCHK(launch_accept(c->tblock, c->tpost, k, c->tstate, c->toutlog, c->tresult, s));
  HIPCHK(hipMemcpyAsync(h + 256, c->tresult, (k + 3) * 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(h + 320, c->tstate, 2 * 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  *a = h[256];
  // internal consistency of the kernel's outputs
  if (h[257] != h[256] + 1 || h[320] != h[257] || h[321] != h[257])
    return fail(SSD_E_HIP, "accept kernel produced inconsistent counters");
  return SSD_OK;
}

ssd_status ssd_time_op(ssd_ctx* c, int32_t op, int32_t layer, int32_t m, int32_t iters, float* avg_us) {
  clear_error();
  if (!c || !avg_us) return fail(SSD_E_ARG, "NULL argument");
  const ssd_cfg& g = c->cfg;
  if (layer < 0 || layer >= g.n_layers) return fail(SSD_E_ARG, "layer out of range");
  if (m < 1 || m > c->lay.R) return fail(SSD_E_ARG, "m outside [1, %d]", c->lay.R);
  if (op == 7 && (size_t)256 * m > (size_t)c->cfg.max_block * (c->cfg.vocab / 16 + 1))
    return fail(SSD_E_ARG, "too many probe workgroups for the sink buffer");
  if (iters < 1) return fail(SSD_E_ARG, "iters < 1");
  if (c->n + m + 1 > g.max_ctx) return fail(SSD_E_CAPACITY, "no room past the committed length");
  if (op < 0 || op > 8) return fail(SSD_E_ARG, "unknown op %d", op);
  if (op == 6 && !c->L[layer].moe) return fail(SSD_E_ARG, "layer %d is not an MoE layer", layer);
  if (op == 6 && c->moe_inject && m > c->moe_inject) return fail(SSD_E_ARG, "m exceeds the injected routing rows");
  if (op == 4 && m > g.max_block) return fail(SSD_E_ARG, "lm_head timing needs m <= max_block");
  const int d = g.d_model, hq = g.n_q_heads, hkv = g.n_kv_heads, hd = g.head_dim, dt = g.dtype;
  hipStream_t s = c->stream;
  // layers of the same kind as `layer`, visited in turn so that consecutive
  // launches stream different weights (as a real pass does) instead of
  // re-reading one matrix that the on-die caches could hold
  std::vector<int> ring;
  for (int i = 0; i < g.n_layers; ++i) {
    const int l = (layer + i) % g.n_layers;
    if (c->L[l].moe == c->L[layer].moe) ring.push_back(l);
  }
  if ((op == 0 || op == 1) && c->L[layer].moe) return fail(SSD_E_ARG, "layer %d is an MoE layer", layer);
  HIPCHK(hipEventRecord(c->ev[EV_A], s));
  for (int it = 0; it < iters; ++it) {
    const int l = ring[it % ring.size()];
    const LayerW& w = c->L[l];
    void* kc = (char*)c->kc + (size_t)l * cache_layer_elems(g) * c->esz;
    void* vc = (char*)c->vc + (size_t)l * cache_layer_elems(g) * c->esz;
    GemmArgs a{};
    int epi = -1;
    switch (op) {
      case 0:
        a.X = c->xn; a.ldx = d; a.W0 = w.w_gate; a.W1 = w.w_up; a.M = m; a.N = w.ffn; a.K = d; a.out = c->act; a.ldo = w.ffn;
        epi = EPI_SWIGLU; break;
      case 1:
        a.X = c->act; a.ldx = w.ffn; a.W0 = w.w_down; a.M = m; a.N = d; a.K = w.ffn; a.y = c->x; a.ldy = d;
        epi = EPI_RESID; break;
      case 2:
        a.X = c->xn; a.ldx = d; a.W0 = w.wq; a.W1 = w.wk; a.W2 = w.wv; a.n0 = hq * hd; a.n1 = hkv * hd; a.M = m;
        a.N = (hq + 2 * hkv) * hd; a.K = d; a.q = c->q; a.kc = kc; a.vc = vc; a.cos_t = c->cos_t; a.sin_t = c->sin_t;
        a.state = c->dstate; a.pos_off = 0; a.hq = hq; a.hkv = hkv; a.hd = hd; a.max_ctx = kv_stride(g);
        epi = EPI_QKV; break;
      case 3:
        a.X = c->att; a.ldx = hq * hd; a.W0 = w.wo; a.M = m; a.N = d; a.K = hq * hd; a.y = c->x; a.ldy = d;
        epi = EPI_RESID; break;
      case 4:
        a.X = c->xn; a.ldx = d; a.W0 = c->lm_head; a.M = m; a.N = g.vocab; a.K = d; a.y = c->logits; a.ldy = g.vocab;
        a.amax_v = c->amax_v; a.amax_i = c->amax_i;
        epi = dt == SSD_BF16 ? EPI_LOGITS : EPI_F32; break;
      default: break;
    }
    if (op == 8) {
      // plain copy of m MiB from the LM head matrix into the attention partial buffer
      const size_t bytes = std::min(std::min((size_t)m << 20, c->lay.part_o_bytes), (size_t)g.vocab * d * c->esz);
      HIPCHK(launch_copy_f32((const float*)c->lm_head, c->part_o, (int)(bytes / 4), s));
    } else if (op == 7) {
      // read probe over the LM head matrix; m = workgroups per CU (x256)
      const size_t bytes = (size_t)g.vocab * d * c->esz;
      HIPCHK(launch_read_probe(c->lm_head, bytes, (unsigned*)c->amax_i, 256 * m, s));
    } else if (op == 6) {
      HIPCHK(launch_moe(dt, moe_args(c, l, m), s));
    } else if (op == 5) {
      AttnArgs at{};
      at.q = c->q; at.kc = kc; at.vc = vc; at.out = c->att; at.part_o = c->part_o; at.part_ml = c->part_ml; at.pstride = c->lay.n_part;
      at.state = c->dstate; at.pos_off = 0; at.M = m; at.R = c->lay.R;
      at.hq = hq; at.hkv = hkv; at.hd = hd; at.max_ctx = kv_stride(g);
      at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
      at.out_p = frag_pass(c, m) ? c->att_p : nullptr;
      HIPCHK(launch_attention(dt, at, (c->n + m + ATT_PT - 1) / ATT_PT, s));
    } else {
      // bf16 GEMMs carry their folded-norm work as in a pass
      if (dt == SSD_BF16 && (op == 0 || op == 2 || op == 4)) fold_in(c, a, 0);
      if (dt == SSD_BF16 && (op == 1 || op == 3)) fold_out(c, a, w.ffn_norm);
      if (frag_pass(c, m)) {   // as a pass of m rows: fragment-order inputs and outputs
        a.Xp = op == 1 ? c->act_p : op == 3 ? c->att_p : c->xn_p;
        if (op == 0) a.out_p = c->act_p;
        if (op == 1 || op == 3) a.xg_out_p = c->xn_p;
      }
      HIPCHK(run_gemm(c, epi, a));
    }
  }
  HIPCHK(hipEventRecord(c->ev[EV_B], s));
  HIPCHK(hipStreamSynchronize(s));
  *avg_us = elapsed(c->ev[EV_A], c->ev[EV_B]) * 1000.f / iters;
  return SSD_OK;
}

}  // extern "C"
