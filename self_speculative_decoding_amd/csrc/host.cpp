// Host-only parts of the C ABI: configuration checks, the canonical weight
// table, workspace layout, the layer-skip mask and the call state machine.
// Nothing here calls HIP, so all of it runs (and is tested) without a GPU.
#include "host.h"

#include <vector>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

namespace ssd {

static thread_local std::string g_err;

ssd_status fail(ssd_status s, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

const char* last_error() { return g_err.c_str(); }
void clear_error() { g_err.clear(); }

bool is_moe_layer(const ssd_cfg& c, int l) { return c.n_experts > 0 && l >= c.n_dense_layers; }

int layer_ffn(const ssd_cfg& c) { return c.n_experts > 0 ? c.dense_ffn : c.ffn_dim; }

std::vector<int64_t> weight_table(const ssd_cfg& c, std::vector<char>* gemm) {
  const int64_t d = c.d_model, hd = c.head_dim, hq = c.n_q_heads, hkv = c.n_kv_heads;
  std::vector<int64_t> t;
  std::vector<char> g;
  auto add = [&](int64_t n, bool is_gemm) { t.push_back(n); g.push_back(is_gemm); };
  add((int64_t)c.vocab * d, false);
  for (int l = 0; l < c.n_layers; ++l) {
    add(d, false);
    add(hq * hd * d, true);
    add(hkv * hd * d, true);
    add(hkv * hd * d, true);
    add(d * hq * hd, true);
    add(d, false);
    if (is_moe_layer(c, l)) {
      const int64_t e = c.n_experts, fe = c.expert_ffn, s = c.n_shared;
      add(e * d, true);
      add(e * fe * d, true);
      add(e * fe * d, true);
      add(e * d * fe, true);
      add(s * fe * d, true);
      add(s * fe * d, true);
      add(s * d * fe, true);
    } else {
      const int64_t f = layer_ffn(c);
      add(f * d, true);
      add(f * d, true);
      add(d * f, true);
    }
  }
  add(d, false);
  add((int64_t)c.vocab * d, true);
  if (c.n_feat > 0) add(d * c.n_feat * d, true);
  if (gemm) *gemm = g;
  return t;
}

int64_t packed_elems(const ssd_cfg& c) {
  if (c.dtype != SSD_BF16) return 0;
  std::vector<char> g;
  const auto t = weight_table(c, &g);
  int64_t n = 0;
  for (size_t i = 0; i < t.size(); ++i)
    if (g[i]) n += t[i];
  return n;
}

ssd_status validate(const ssd_cfg* cp) {
  if (!cp) return fail(SSD_E_ARG, "cfg is NULL");
  const ssd_cfg& c = *cp;
  if (c.n_layers < 1 || c.d_model < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 1 || c.vocab < 2)
    return fail(SSD_E_ARG, "non-positive model dimension");
  if (c.dtype != SSD_F32 && c.dtype != SSD_BF16) return fail(SSD_E_ARG, "dtype must be 0 (f32) or 1 (bf16)");
  if (c.n_q_heads % c.n_kv_heads) return fail(SSD_E_ARG, "n_q_heads %% n_kv_heads != 0");
  const int G = c.n_q_heads / c.n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return fail(SSD_E_UNSUPPORTED, "query heads per KV head must be 1, 2 or 4");
  if (c.head_dim != 64 && c.head_dim != 128) return fail(SSD_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 1.f)) return fail(SSD_E_ARG, "rms_eps/rope_theta out of range");
  if (c.max_block < 1 || c.max_block > SSD_MAX_BLOCK) return fail(SSD_E_ARG, "max_block must be in [1, %d]", SSD_MAX_BLOCK);
  if (c.prefill_chunk < 16 || c.prefill_chunk > 256 || c.prefill_chunk % 16)
    return fail(SSD_E_ARG, "prefill_chunk must be a multiple of 16 in [16, 256]");
  // the attention combine holds one partition of kAttPT keys per lane of a 128-lane workgroup
  if (c.max_ctx < 2 || c.max_ctx > 128 * kAttPT) return fail(SSD_E_ARG, "max_ctx must be in [2, %d]", 128 * kAttPT);
  if (c.n_experts < 0 || c.n_shared < 0 || c.n_dense_layers < 0 || c.n_feat < 0)
    return fail(SSD_E_ARG, "negative count");
  if (c.n_experts > 0) {
    if (c.n_experts > 64) return fail(SSD_E_UNSUPPORTED, "at most 64 routed experts");
    if (c.dtype != SSD_BF16) return fail(SSD_E_UNSUPPORTED, "MoE layers run in bf16");
    if (c.n_experts % 16) return fail(SSD_E_UNSUPPORTED, "n_experts must be a multiple of 16");
    if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > 8) return fail(SSD_E_ARG, "top_k must be in [1, min(8, n_experts)]");
    if (c.expert_ffn < 1) return fail(SSD_E_ARG, "expert_ffn must be positive");
    if (c.n_shared > 8) return fail(SSD_E_UNSUPPORTED, "at most 8 shared experts");
    if (c.n_dense_layers > c.n_layers) return fail(SSD_E_ARG, "n_dense_layers > n_layers");
    if (c.n_dense_layers > 0 && c.dense_ffn < 1) return fail(SSD_E_ARG, "dense_ffn must be positive");
  } else if (c.ffn_dim < 1) {
    return fail(SSD_E_ARG, "ffn_dim must be positive");
  }
  if (c.n_feat > SSD_MAX_FEAT) return fail(SSD_E_ARG, "n_feat > %d", SSD_MAX_FEAT);
  for (int i = 0; i < c.n_feat; ++i) {
    if (c.feat_layers[i] < 0 || c.feat_layers[i] >= c.n_layers) return fail(SSD_E_ARG, "feat_layers[%d] out of range", i);
    if (i && c.feat_layers[i] <= c.feat_layers[i - 1]) return fail(SSD_E_ARG, "feat_layers must increase");
    if (is_moe_layer(c, c.feat_layers[i])) return fail(SSD_E_UNSUPPORTED, "feature tap on an MoE layer");
  }
  // kernel shape requirements
  if (c.d_model % 4 || c.d_model > 16384) return fail(SSD_E_UNSUPPORTED, "d_model must be a multiple of 4 and <= 16384");
  if (c.vocab > 16 * 16384) return fail(SSD_E_UNSUPPORTED, "vocab must be <= 262144");
  const int64_t qo = (int64_t)c.n_q_heads * c.head_dim;
  const int f = layer_ffn(c);
  if (c.dtype == SSD_BF16) {
    auto k32 = [](int64_t v) { return v % 64 == 0; };   // GEMM K runs in 64-element chunks
    auto n16 = [](int64_t v) { return v % 16 == 0; };
    if (!k32(c.d_model) || !k32(qo)) return fail(SSD_E_UNSUPPORTED, "bf16: d_model and heads*head_dim must be multiples of 64");
    if (!n16(c.vocab)) return fail(SSD_E_UNSUPPORTED, "bf16: vocab must be a multiple of 16");
    if (f > 0 && (!k32(f))) return fail(SSD_E_UNSUPPORTED, "bf16: FFN width must be a multiple of 64");
    if (c.n_experts > 0 && !k32(c.expert_ffn)) return fail(SSD_E_UNSUPPORTED, "bf16: expert_ffn must be a multiple of 64");
  } else {
    if (c.d_model % 2 || c.vocab % 2 || qo % 2) return fail(SSD_E_UNSUPPORTED, "f32: d_model, vocab, heads*head_dim must be even");
    if (c.n_experts > 0 && c.expert_ffn % 2) return fail(SSD_E_UNSUPPORTED, "f32: expert_ffn must be even");
  }
  return SSD_OK;
}

static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

TracePoints trace_points(const ssd_cfg& c) {
  TracePoints t;
  const size_t esz = c.dtype == SSD_BF16 ? 2 : 4, d = c.d_model, qo = (size_t)c.n_q_heads * c.head_dim;
  size_t f = (size_t)layer_ffn(c);   // dense activation, or the MoE layers' [slot][expert_ffn]
  if (c.n_experts > 0 && (size_t)(c.top_k + c.n_shared) * c.expert_ffn > f) f = (size_t)(c.top_k + c.n_shared) * c.expert_ffn;
  const size_t rows[6] = {d * esz, qo * esz, qo * esz, d * 4, d * esz, f * esz};
  size_t off = 0;
  for (int i = 0; i < 6; ++i) {
    t.off[i] = off;
    t.row[i] = rows[i];
    off = up256(off + rows[i] * c.max_block);
  }
  t.layer = off;
  t.total = (size_t)c.n_layers * t.layer + up256(d * esz * c.max_block);
  return t;
}

bool compute_layout(const ssd_cfg& c, Layout& L) {
  if (validate(&c) != SSD_OK) return false;
  const size_t esz = c.dtype == SSD_BF16 ? 2 : 4;
  const size_t d = c.d_model, hd = c.head_dim, hq = c.n_q_heads, hkv = c.n_kv_heads;
  int R = c.max_block > c.prefill_chunk ? c.max_block : c.prefill_chunk;
  R = (R + 15) / 16 * 16;
  L.R = R;
  L.n_part = (c.max_ctx + kAttPT - 1) / kAttPT;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = up256(off + bytes); return o; };
  const size_t cache = (size_t)c.n_layers * hkv * ((size_t)L.n_part * kAttPT) * hd * esz;   // rows padded to whole partitions
  L.kc = take(cache);
  L.vc = take(cache);
  L.x = take((size_t)R * d * 4);
  L.xn = take((size_t)R * d * esz);
  L.ss = take((size_t)R * (d / 8) * 4);   // folded-norm partial sums of squares (tiles of >= 8 columns)
  L.q = take((size_t)R * hq * hd * esz);
  L.att = take((size_t)R * hq * hd * esz);
  size_t fact = (size_t)layer_ffn(c);
  if (c.n_experts > 0) {
    const size_t fm = (size_t)(c.top_k + c.n_shared) * c.expert_ffn;
    if (fm > fact) fact = fm;
  }
  L.act = take((size_t)R * fact * esz);
  L.logits = take((size_t)c.max_block * c.vocab * 4);
  L.amax_v = take((size_t)c.max_block * (c.vocab / 16 + 1) * 4);
  L.trace = take((size_t)c.n_layers * c.max_block * d * 4);
  L.trace_pts = take(trace_points(c).total);
  // exit-state cache of an early-exit draft: residual and its sums of squares
  // per block row after the draft's last layer
  L.exit_x = take((size_t)c.max_block * d * 4);
  L.exit_ss = take((size_t)c.max_block * (d / 8) * 4);
  // speculative sampling: the draft steps' logits rows, test-cycle outputs
  L.dlog = take((size_t)c.max_block * c.vocab * 4);
  L.tout = take((size_t)kTestCycles * (SSD_MAX_BLOCK + 2) * 4);
  L.smp_nch = ((size_t)c.vocab + kSmpChunk - 1) / kSmpChunk;   // sampling scratch
  L.smp_stats = take((size_t)kSmpRows * L.smp_nch * 8);
  L.smp_csum = take(2 * L.smp_nch * 4);
  L.smp_ctl = take(kSmpCtlBytes);
  L.amax_i = take((size_t)c.max_block * (c.vocab / 16 + 1) * 4);
  L.part_o_bytes = (size_t)L.n_part * R * hq * hd * 4;
  L.part_o = take(L.part_o_bytes);
  L.part_ml = take((size_t)L.n_part * R * hq * 2 * 4);
  L.rope_cos = take((size_t)c.max_ctx * (hd / 2) * 4);
  L.rope_sin = take((size_t)c.max_ctx * (hd / 2) * 4);
  L.block = take(SSD_MAX_BLOCK * 4);
  L.post = take(SSD_MAX_BLOCK * 4);
  L.toks = take((size_t)R * 4);
  L.state = take(16 * 4);
  L.result = take((SSD_MAX_BLOCK + 2) * 4);
  L.outlog = take(((size_t)c.max_ctx + SSD_MAX_BLOCK) * 4);
  L.tblock = take(SSD_MAX_BLOCK * 4);
  L.tpost = take(SSD_MAX_BLOCK * 4);
  L.tstate = take(16 * 4);
  L.tresult = take((SSD_MAX_BLOCK + 2) * 4);
  L.toutlog = take((SSD_MAX_BLOCK + 2) * 4);
  if (c.n_feat > 0) {
    L.tap = take((size_t)c.max_block * c.n_feat * d * esz);
    L.feat = take((size_t)c.max_block * d * esz);
  }
  if (c.n_experts > 0) {
    const size_t slots = (size_t)c.top_k + c.n_shared;
    L.m_rlogits = take((size_t)R * c.n_experts * 4);
    L.m_ids = take((size_t)R * c.top_k * 4);
    L.m_gates = take((size_t)R * c.top_k * 4);
    L.m_inject = take((size_t)c.n_layers * R * c.top_k * 4);
    L.m_slot_out = take((size_t)R * slots * d * 4);
    const size_t max_units = (size_t)R * c.top_k + (size_t)((R + 15) / 16) * c.n_shared;
    L.m_groups = take((16 + max_units * 18) * 4);
    L.m_union = take((size_t)c.n_layers * 4);
    L.m_rstd = take((size_t)R * 4);
  }
  if (c.dtype == SSD_BF16 && c.n_experts == 0) {   // fragment-order copies of the dense GEMM inputs
    L.frag = true;
    L.xn_p = take((size_t)kFragRows * d * 2);
    L.att_p = take((size_t)kFragRows * hq * hd * 2);
    L.act_p = take((size_t)kFragRows * c.ffn_dim * 2);
    if (c.n_feat > 0) L.tap_p = take((size_t)kFragRows * c.n_feat * d * 2);
  }
  L.wpack = take((size_t)packed_elems(c) * 2);   // bf16 GEMM weights in the packed tile layout
  L.total = off;
  return true;
}

ssd_status check_transition(int32_t state, int32_t op, int32_t* next) {
  int n = -1;
  switch (op) {
    case SSD_OP_PREFILL: if (state == SSD_ST_LOADED) n = SSD_ST_READY; break;
    case SSD_OP_DRAFT: if (state == SSD_ST_READY) n = SSD_ST_DRAFTED; break;
    case SSD_OP_VERIFY: if (state == SSD_ST_DRAFTED) n = SSD_ST_VERIFIED; break;
    case SSD_OP_VERIFY_BLOCK: if (state == SSD_ST_READY || state == SSD_ST_DRAFTED) n = SSD_ST_VERIFIED; break;
    case SSD_OP_ACCEPT: if (state == SSD_ST_VERIFIED) n = SSD_ST_READY; break;
    case SSD_OP_RESET:
      if (state >= SSD_ST_LOADED && state <= SSD_ST_VERIFIED) n = SSD_ST_LOADED;
      break;
    default: return fail(SSD_E_ARG, "unknown operation %d", op);
  }
  if (n < 0) {
    static const char* names[] = {"LOADED", "READY", "DRAFTED", "VERIFIED"};
    static const char* ops[] = {"prefill", "draft", "verify", "verify(block)", "accept_rollback", "reset"};
    return fail(SSD_E_STATE, "%s not allowed in state %s", ops[op],
                state >= 0 && state <= 3 ? names[state] : "?");
  }
  if (next) *next = n;
  return SSD_OK;
}

ssd_status skip_mask(int32_t n_layers, double frac, uint8_t* mask) {
  if (n_layers < 1 || !mask) return fail(SSD_E_ARG, "n_layers < 1 or mask is NULL");
  if (!(frac >= 0.0 && frac <= 1.0)) return fail(SSD_E_ARG, "skip fraction must be in [0, 1]");
  // round half to even on the same double product (nearbyint under the default rounding mode)
  long n_skip = (long)std::nearbyint((double)n_layers * frac);
  if (n_skip < 1) n_skip = 1;
  if (n_skip > n_layers) n_skip = n_layers;
  const long start = (n_layers - n_skip) / 2;
  for (int l = 0; l < n_layers; ++l) mask[l] = (l >= start && l < start + n_skip) ? 1 : 0;
  return SSD_OK;
}

}  // namespace ssd

// ---- exported host-only entry points ---------------------------------------

extern "C" {

ssd_status ssd_validate_cfg(const ssd_cfg* cfg) {
  ssd::clear_error();
  return ssd::validate(cfg);
}

int32_t ssd_n_weights(const ssd_cfg* cfg) {
  if (ssd::validate(cfg) != SSD_OK) return -1;
  return (int32_t)ssd::weight_table(*cfg).size();
}

int64_t ssd_weight_numel(const ssd_cfg* cfg, int32_t i) {
  if (ssd::validate(cfg) != SSD_OK) return -1;
  auto t = ssd::weight_table(*cfg);
  if (i < 0 || i >= (int32_t)t.size()) return -1;
  return t[i];
}

int32_t ssd_weight_retained(const ssd_cfg* cfg, int32_t i) {
  if (ssd::validate(cfg) != SSD_OK) return -1;
  std::vector<char> g;
  auto t = ssd::weight_table(*cfg, &g);
  if (i < 0 || i >= (int32_t)t.size()) return -1;
  return cfg->dtype == SSD_BF16 && g[i] ? 0 : 1;
}

int64_t ssd_workspace_bytes(const ssd_cfg* cfg) {
  ssd::Layout L;
  if (!cfg || !ssd::compute_layout(*cfg, L)) return -1;
  return (int64_t)L.total;
}

ssd_status ssd_skip_mask(int32_t n_layers, double frac, uint8_t* mask) {
  ssd::clear_error();
  return ssd::skip_mask(n_layers, frac, mask);
}

ssd_status ssd_select_k(const double* t_verify, int32_t kmax, double t_draft, double t_cycle, double alpha,
                        int32_t* k_best, double* rate) {
  ssd::clear_error();
  if (!t_verify || !k_best || !rate) return ssd::fail(SSD_E_ARG, "NULL argument");
  if (kmax < 0 || kmax > SSD_MAX_BLOCK - 1) return ssd::fail(SSD_E_ARG, "kmax=%d outside [0, %d]", kmax, SSD_MAX_BLOCK - 1);
  if (!(alpha >= 0.0 && alpha <= 1.0)) return ssd::fail(SSD_E_ARG, "alpha must be in [0, 1]");
  if (!(t_draft > 0.0) || !(t_cycle >= 0.0)) return ssd::fail(SSD_E_ARG, "t_draft must be > 0 and t_cycle >= 0");
  for (int k = 0; k <= kmax; ++k)
    if (!(t_verify[k] > 0.0)) return ssd::fail(SSD_E_ARG, "t_verify[%d] must be > 0", k);
  int best = 0;
  double best_rate = -1.0, e = 0.0, ak = 1.0;
  for (int k = 0; k <= kmax; ++k) {
    e += ak;   // E_k = 1 + alpha + ... + alpha^k
    ak *= alpha;
    const double r = e / (k * t_draft + t_verify[k] + t_cycle);
    if (r > best_rate) {
      best_rate = r;
      best = k;
    }
  }
  *k_best = best;
  *rate = best_rate;
  return SSD_OK;
}

ssd_status ssd_knapsack_skip(const int32_t* cost, const double* value, int32_t n, int64_t budget, uint8_t* mask,
                             double* kept_value) {
  ssd::clear_error();
  if (!cost || !value || !mask || !kept_value) return ssd::fail(SSD_E_ARG, "NULL argument");
  if (n < 1 || budget < 0) return ssd::fail(SSD_E_ARG, "n_layers must be >= 1 and budget >= 0");
  if ((int64_t)n * (budget + 1) > ((int64_t)1 << 26)) return ssd::fail(SSD_E_ARG, "n_layers * (budget + 1) too large");
  for (int i = 0; i < n; ++i)
    if (cost[i] < 0) return ssd::fail(SSD_E_ARG, "cost[%d] < 0", i);
  const size_t B = (size_t)budget + 1;
  // best[b]: best value of the layers seen so far with total cost <= b;
  // take[i*B + b]: layer i kept in that optimum
  std::vector<double> best(B, 0.0);
  std::vector<uint8_t> take((size_t)n * B, 0);
  for (int i = 0; i < n; ++i) {
    const size_t c = (size_t)cost[i];
    for (size_t b = B; b-- > 0;) {
      if (b < c) break;
      const double v = best[b - c] + value[i];
      if (v > best[b]) {
        best[b] = v;
        take[(size_t)i * B + b] = 1;
      }
    }
  }
  size_t b = B - 1;
  for (int i = n - 1; i >= 0; --i) {
    if (take[(size_t)i * B + b]) {
      mask[i] = 0;
      b -= (size_t)cost[i];
    } else {
      mask[i] = 1;
    }
  }
  *kept_value = best[B - 1];
  return SSD_OK;
}

ssd_status ssd_check_transition(int32_t state, int32_t op, int32_t* next_state) {
  ssd::clear_error();
  return ssd::check_transition(state, op, next_state);
}

const char* ssd_strerror(ssd_status s) {
  switch (s) {
    case SSD_OK: return "ok";
    case SSD_E_ARG: return "invalid argument";
    case SSD_E_STATE: return "call not allowed in the current state";
    case SSD_E_CAPACITY: return "KV cache capacity exceeded";
    case SSD_E_HIP: return "HIP runtime error";
    case SSD_E_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* ssd_last_error(void) { return ssd::last_error(); }

}  // extern "C"
