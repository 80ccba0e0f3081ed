// Host-only helpers shared by host.cpp and runtime.hip (no HIP calls).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "ssd.h"

namespace ssd {

constexpr int kAttPT = 64;   // attention key partition width (kernels.h: ATT_PT)
// Passes of kFragMinM..kFragRows rows of dense bf16 models also keep their
// GEMM inputs in fragment order (frag_index in device.h): two row tiles.
constexpr int kFragMinM = 5, kFragRows = 32;
constexpr int kTestCycles = 4096;   // sampling test cycles per output copy
// sampling scratch (kernels.h: SMP_CHUNK, SMP_ROWS, SMP_CTL_BYTES)
constexpr int kSmpChunk = 2048, kSmpRows = 63, kSmpCtlBytes = 64;

// Byte offsets of every workspace buffer (256-byte aligned).
struct Layout {
  size_t kc = 0, vc = 0, x = 0, xn = 0, ss = 0, q = 0, att = 0, act = 0, logits = 0;
  size_t part_o = 0, part_ml = 0, rope_cos = 0, rope_sin = 0;
  size_t block = 0, post = 0, toks = 0, state = 0, result = 0, outlog = 0;
  size_t tblock = 0, tpost = 0, tstate = 0, tresult = 0, toutlog = 0;
  size_t tap = 0, feat = 0, amax_v = 0, amax_i = 0, trace = 0, trace_pts = 0, wpack = 0, exit_x = 0, exit_ss = 0, dlog = 0, tout = 0;
  size_t smp_stats = 0, smp_csum = 0, smp_ctl = 0, smp_nch = 0;
  size_t m_rlogits = 0, m_ids = 0, m_gates = 0, m_inject = 0, m_slot_out = 0, m_groups = 0, m_union = 0, m_rstd = 0;
  size_t xn_p = 0, att_p = 0, act_p = 0, tap_p = 0;   // fragment-order GEMM inputs (frag = true)
  bool frag = false;
  size_t total = 0;
  int R = 0;        // rows per pass (multiple of 16)
  int n_part = 0;   // attention partitions covering max_ctx
  size_t part_o_bytes = 0;
};

// Stored operands of every layer of a traced pass (SSD_OPT_TRACE): per layer
// six points of up to max_block rows each: the QKV input, q after RoPE, the
// attention output, the residual after the attention block (float32), the
// gate/up input and the SwiGLU activation; then the LM head's input.
struct TracePoints {
  size_t off[6] = {};     // byte offset of each point inside a layer record
  size_t row[6] = {};     // bytes per row of each point
  size_t layer = 0;       // bytes per layer record
  size_t total = 0;       // all layers + the head input
};
TracePoints trace_points(const ssd_cfg& c);

ssd_status fail(ssd_status s, const char* fmt, ...);
const char* last_error();
void clear_error();
ssd_status validate(const ssd_cfg* c);
bool compute_layout(const ssd_cfg& c, Layout& L);
// element counts of the weight tensors in ssd_load order; gemm (optional)
// flags the matrices the bf16 GEMMs read (packed at load)
std::vector<int64_t> weight_table(const ssd_cfg& c, std::vector<char>* gemm = nullptr);
int64_t packed_elems(const ssd_cfg& c);
bool is_moe_layer(const ssd_cfg& c, int l);
int layer_ffn(const ssd_cfg& c);
ssd_status check_transition(int32_t state, int32_t op, int32_t* next);
ssd_status skip_mask(int32_t n_layers, double frac, uint8_t* mask);

}  // namespace ssd
