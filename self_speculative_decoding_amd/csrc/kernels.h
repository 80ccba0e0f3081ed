// Internal interface between the runtime (runtime.hip) and the gfx950 kernels
// (kernels.hip).  Not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Key partition width of the decode attention: partitions are anchored at
// absolute positions [p*ATT_PT, (p+1)*ATT_PT), so a row's reduction order
// depends only on its own position, never on the block it is verified in.
constexpr int ATT_PT = 64;
constexpr int ROW_TILE = 16;   // rows per MFMA tile / attention row tile

enum Epi {
  EPI_F32 = 0,     // y[m*ldy + n] = acc                         (logits)
  EPI_RESID = 1,   // y[m*ldy + n] += acc; optional bf16 tap of the new value
  EPI_SWIGLU = 2,  // act[m*ldo + n] = silu(acc_gate) * acc_up   (W0 gate, W1 up)
  EPI_QKV = 3,     // RoPE on q,k; q -> q buffer; k,v -> KV cache at their positions
  EPI_STORE = 4,   // out[m*ldo + n] = acc in the activation type (feature fc)
  EPI_MOE = 5,     // per-row routed/shared expert output accumulation (see moe kernels)
  EPI_LOGITS = 6,  // EPI_F32 plus per-16-column (max, lowest index) pairs for the argmax
};

struct GemmArgs {
  const void* X;              // activations [M, K], row stride ldx (elements)
  int ldx;
  const void* Xp;             // optional: the same activations in fragment order (frag_index), read instead of X
                              // by one-tile-row launches
  const void* W0;             // weights [rows, K] row-major
  const void* W1;
  const void* W2;
  int n0, n1;                 // rows of W0 and W1 (QKV: q rows, k rows)
  int M, N, K;                // N = output columns (SwiGLU: intermediate width)
  float* y;                   // f32 output / residual
  int ldy;
  void* out;                  // activation-typed output (SwiGLU act, STORE)
  int ldo;
  void* tap;                  // RESID: optional copy of the new residual (activation type)
  int ldtap;
  void* tap_p;                // RESID: optional fragment-order copy of the tap: column tap_col + n of [M, ldtap]
  int tap_col;
  void* out_p;                // SWIGLU: optional fragment-order copy of out ([M, N])
  // QKV epilogue
  void* q;                    // [M, hq*hd]
  void* kc;                   // this layer's K cache [hkv][max_ctx][hd]
  void* vc;                   // this layer's V cache, transposed: [hkv][hd][max_ctx]
  const float* cos_t;         // [positions][hd/2]
  const float* sin_t;
  const int* state;           // state[0] = committed length n
  int pos_off;                // row r sits at position state[0] + pos_off + r
  int hq, hkv, hd, max_ctx;   // max_ctx: positions per cache row (a multiple of 64)
  // LOGITS epilogue: per-tile argmax partials [M][N/16]
  float* amax_v;
  int* amax_i;
  // RMSNorm folded into the GEMMs (bf16 models).  A consumer GEMM (QKV,
  // gate/up, LM head) reads X = bf16(x * gain) and scales its float
  // accumulator by rstd = 1/sqrt(mean(x^2) + eps), summing the partial sums
  // of squares ss_in [M][nss] (nss a multiple of 4) the producer left.  The
  // producer (residual epilogue) writes one partial per column tile (ss_out
  // [M][N/TW]) and the next consumer's input xg_out = bf16(x_new * gain_next)
  // [M][N].
  const float* ss_in;
  int nss;
  float eps;
  float* ss_out;
  void* xg_out;
  const void* gain_next;
  void* xg_out_p;             // optional fragment-order copy of xg_out ([M, N])
  // set by the launcher only: a 1-D launch of remap_gx x remap_rb workgroups
  // of the multi-row-tile kernel mapped XCD-aware (see gemm.hip); 0 otherwise
  int remap_gx, remap_rb;
  // long passes: fewest workgroups a wider column group may leave (0: the
  // built-in SSD_TILE_WG_MIN); never changes a result
  int tile_wg_min;
};

struct AttnArgs {
  const void* q;              // [M, hq*hd]
  const void* kc;             // [hkv][max_ctx][hd]
  const void* vc;             // [hkv][hd][max_ctx]
  void* out;                  // [M, hq*hd]
  void* out_p;                // optional fragment-order copy of out (bf16 only)
  float* part_o;              // [R][hq][pstride][hd]: one row-head's partitions contiguous
  float* part_ml;             // [R][hq][pstride][2]
  const int* state;
  int pos_off, M, R, hq, hkv, hd, max_ctx;   // max_ctx: positions per cache row (multiple of 64)
  int n_part;                 // partitions launched (set by launch_attention)
  int pstride;                // partition slots per (row, head) in part_o / part_ml (>= n_part)
  int xcd;                    // set by the launcher: 1-D XCD-affine grids (attn_xcd_map)
  float scale_log2;           // log2(e) / sqrt(hd)
};

// dtype: 0 = f32, 1 = bf16 (uint16 bit patterns)
hipError_t launch_embed(int dtype, const int* tok, const void* E, float* x, int d, int M, hipStream_t s);
// bf16 embedding that also leaves the folded-RMSNorm inputs of the first layer:
// xg = bf16(x * gain) and sums of squares over runs of ssw columns (16, 10 or 8), ss [M][d/ssw];
// xgp (optional): a fragment-order copy of xg (frag_index)
hipError_t launch_embed_norm(const int* tok, const void* E, float* x, int d, int M, const void* gain, void* xg,
                             float* ss, int ssw, hipStream_t s, void* xgp = nullptr);
hipError_t launch_rmsnorm(int dtype, const float* x, int ldx, const void* g, void* y, int ldy, int d,
                          float eps, int M, hipStream_t s);
hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s);
hipError_t launch_attention(int dtype, const AttnArgs& a, int n_part, hipStream_t s);
hipError_t launch_argmax(const float* logits, int V, int ld, int* out, int M, hipStream_t s);
hipError_t launch_argmax_tiles(const float* pv, const int* pi, int nt, int* out, int M, hipStream_t s);
hipError_t launch_accept(int* block, const int* post, int k, int* state, int* outlog, int* result,
                         hipStream_t s);
hipError_t launch_set_state(int* state, int idx, int value, hipStream_t s);
hipError_t launch_read_probe(const void* src, size_t bytes, unsigned* sink, int blocks, hipStream_t s);
hipError_t launch_copy_tokens(const int* src, int* dst, int n, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t s);
// xg[m][n] = bf16(x[m][n] * g[n]) for M rows of d (the folded-norm input); xgp as in launch_embed_norm
hipError_t launch_scale_bf16(const float* x, const void* g, void* xg, int d, int M, hipStream_t s,
                             void* xgp = nullptr);

// MoE (routed experts + shared experts)
struct MoeArgs {
  const void* X;              // input rows [M, d]: bf16(x * ffn_norm gain) with ss_in set, else normalised
  const float* ss_in;         // folded RMSNorm (see GemmArgs): router and expert gate/up products of row m
  int nss;                    // are scaled by its 1/rms, from these nss partials per row
  float eps;
  float* rstd;                // [M] scratch: each token's 1/rms (written by the routing kernel)
  int M, d, E, top_k, fe, n_shared;
  const void* router;         // [E, d]
  const void* eg; const void* ed;   // packed: per expert gate/up interleaved [fe x d], down [d x fe]
  const void* sg; const void* sd;   // shared experts, same layout
  float* rlogits;             // [M, E] f32
  int* ids;                   // [M, top_k]  (router choice, or injected)
  float* gates;               // [M, top_k]
  const int* inject;          // [M, top_k] injected ids or null
  void* act;                  // [M, top_k + S, fe] activation type
  float* slot_out;            // [M, top_k + S, d] f32
  float* resid;               // [M, d] residual (+= combined output)
  int* groups;                // dedup work list (see kernels)
  int* union_out;             // [1] union size of this pass
  int dedup;
  // folded RMSNorm of the next GEMM (see GemmArgs): written when ss_out != 0
  float* ss_out;              // [M, d/ssw]: sums of squares over runs of ssw columns
  int ssw;                    // columns per combine run: 16, 10 or 8, dividing d (launch_moe checks)
  void* xg_out;               // [M, d] bf16(x * gain_next)
  const void* gain_next;      // [d]
};
hipError_t launch_moe(int dtype, const MoeArgs& a, hipStream_t s);

// Speculative sampling (sampling.hip).  Logits rows are float32, ld apart;
// T > 0 the temperature; the cycle counter is state[2].  Each call is three
// launches over chunks of SMP_CHUNK columns; SmpBufs is their scratch:
// stats [SMP_ROWS][nch_max] float pairs, csum [2 * nch_max], ctl SMP_CTL_BYTES.
constexpr int SMP_CHUNK = 2048;
constexpr int SMP_ROWS = 63;       // 2 * 32 - 1: target and draft rows of the largest cycle
constexpr int SMP_CTL_BYTES = 64;
struct SmpBufs {
  void* stats;
  float* csum;
  void* ctl;
  int nch_max;   // chunks of the widest row
};
// One decode-loop cycle: drafts block[1..k], target rows tl[0..k], draft rows
// dl[0..k-1]; commits a+1 tokens like the greedy accept (outlog may be null);
// trial_out (or null) receives a, the emitted tokens and -1 up to k+2 entries.
hipError_t launch_spec_accept(const float* tl, const float* dl, int ld, int V, int k, float T, uint64_t seed,
                              int* block, int* state, int* outlog, int* result, int* trial_out, const SmpBufs& b,
                              hipStream_t s);
// draft step `slot`: block[slot + 1] ~ softmax(l / T); the row is copied to keep (or not, if null)
hipError_t launch_draft_sample(const float* l, int V, float T, uint64_t seed, int* block, const int* state, int slot,
                               float* keep, const SmpBufs& b, hipStream_t s);
// first token after a sampled prefill (replaces its argmax in block[0] and the log)
hipError_t launch_first_sample(const float* l, int V, float T, uint64_t seed, int* block, int* state, int* outlog,
                               const SmpBufs& b, hipStream_t s);

// Packing of a row-major bf16 weight [N, K] into the tile layout the bf16
// GEMMs stream (see device.h).  mode 0: rows of src0 in order; mode 1: the
// QKV GEMM's rows gathered from src0 = wq, src1 = wk, src2 = wv; pair: the
// tiles of src0 and src1 (same shape) interleaved one by one (gate/up).
struct PackArgs {
  const void* src0; const void* src1; const void* src2;
  void* dst;
  int N, K, mode, pair, hq, hkv, hd;
  int tw;   // rows per tile (0: 16); mode 0: N % tw == 0; mode 1: 16 or 12 (qkv_col_map)
};

// Compute units of one MI355X: the bf16 GEMMs give every workgroup the same
// weight bytes, so a launch is balanced when its tile count spreads evenly.
constexpr int NUM_CU = 256;
// Rows per packed tile of a dense SwiGLU gate/up weight with N output
// columns: 16, or 14 when that divides N and lowers the largest per-CU share
// of tile bytes (ceil(tiles / NUM_CU) tiles of w rows each).  A function of N
// only; the packing and the GEMM launch both call it.
inline int swiglu_tile_width(int N) {
  if (N % 14 != 0) return 16;
  const long w16 = (long)((N / 16 + NUM_CU - 1) / NUM_CU) * 16;
  const long w14 = (long)((N / 14 + NUM_CU - 1) / NUM_CU) * 14;
  return w14 < w16 ? 14 : 16;
}
// Rows per packed tile of the QKV weight ((hq + 2 hkv) x hd output columns):
// 16, or 12 by the same rule.
inline int qkv_tile_width(int hq, int hkv, int hd) {
  const int N = (hq + 2 * hkv) * hd;
  if (N % 12 != 0) return 16;
  const long w16 = (long)((N / 16 + NUM_CU - 1) / NUM_CU) * 16;
  const long w12 = (long)((N / 12 + NUM_CU - 1) / NUM_CU) * 12;
  return w12 < w16 ? 12 : 16;
}

// Rows per packed tile of the weights whose GEMM adds into the residual
// stream (o projection and down, N = d): 16, 10 or 8, whichever divides N
// into a multiple of 4 tiles with the smallest largest per-CU share (ties to
// the wider tile).  d = 2560 gives 256 tiles of 10 rows instead of 160 of
// 16, so no CU idles.  The folded norm's sums of squares come one per tile
// of these GEMMs: every producer of them writes d / resid_tile_width(d)
// partials per row, each over that many consecutive columns.
inline int resid_tile_width(int N) {
  int best = 16;
  long best_share = (long)((N / 16 + NUM_CU - 1) / NUM_CU) * 16;
  for (int w : {10, 8}) {
    if (N % w != 0 || (N / w) % 4 != 0) continue;
    const long share = (long)((N / w + NUM_CU - 1) / NUM_CU) * w;
    if (share < best_share) {
      best = w;
      best_share = share;
    }
  }
  return best;
}

// Output column of lane c (c < 16) in column tile t of the packed QKV weight
// ([q heads | k heads | v heads], hd dims each) with tw = 16 or 12 columns
// per tile.  kind 0: the first element (dim i < hd/2) of a RoPE pair
// (i, i + hd/2) of a q or k head, whose second element sits on lane c + tw/2;
// kind 1: the second element of a pair, or a lane past the tile (c >= tw);
// kind 2: a V column.  tw = 16 (hd a multiple of 16): dims 8jj..8jj+7 and
// hd/2 + 8jj..+7 of one head.  tw = 12: six whole pairs, pairs numbered
// head-major over the q and k heads, then the V columns in order.
struct QkvCol {
  int head, dim, kind;
};
__host__ __device__ inline QkvCol qkv_col_map(int tw, int t, int c, int hq, int hkv, int hd) {
  const int half = hd >> 1;
  QkvCol r{0, 0, 1};
  if (c >= tw) return r;
  if (tw == 16) {
    const int col0 = t * 16, head = col0 / hd, jj = (col0 % hd) / 16;
    r.head = head;
    if (head < hq + hkv) {
      r.dim = c < 8 ? 8 * jj + c : half + 8 * jj + (c - 8);
      r.kind = c < 8 ? 0 : 1;
    } else {
      r.dim = 16 * jj + c;
      r.kind = 2;
    }
    return r;
  }
  const int pw = tw / 2;                     // pairs per tile
  const int np = (hq + hkv) * half;          // RoPE pairs in all
  const int h = c / pw, q = c % pw;
  int rot = np - pw * t;                     // pairs in this tile
  rot = rot < 0 ? 0 : (rot > pw ? pw : rot);
  if (q < rot) {
    const int p = pw * t + q;
    r.head = p / half;
    r.dim = p % half + h * half;
    r.kind = h == 0 ? 0 : 1;
  } else {
    const int before = tw * t - 2 * (pw * t < np ? pw * t : np);   // V columns in earlier tiles
    const int v = before + h * (pw - rot) + (q - rot);
    r.head = hq + hkv + v / hd;
    r.dim = v % hd;
    r.kind = 2;
  }
  return r;
}
hipError_t launch_pack(const PackArgs& p, hipStream_t s);

}  // namespace ssd
