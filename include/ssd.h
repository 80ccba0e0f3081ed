/*
 * ssd.h - C ABI of the MI355X greedy self-speculative decoding library (libssd.so).
 *
 * The library runs one decoder-only transformer on one AMD MI355X (gfx950) and
 * exposes the speculative decode step the way the method states it:
 *
 *   prompt -> prefill -> repeat { draft k tokens through a subset of the layers
 *   (sharing the KV cache) -> verify the k+1 block tokens in one pass through all
 *   layers -> accept the longest matching prefix plus the verifier's next token
 *   -> cut the KV cache back to the committed length }.
 *
 * Sources: LayerSkip summary page (4.3.1 self-drafting, 4.3.2 self-verification,
 * 4.3.3 reusing the cache); MLX layer-skip blog ("Code": the middle-layer skip
 * draft, lossless greedy check); mlx-dflash README ("Architecture": block verify
 * and greedy cumulative-product accept; "Apple Silicon Optimizations": one host
 * synchronisation per step, draft cache cropped on rejection); speculative
 * decoding for MoE models (abstract: per-slot and deduplicated expert reads).
 *
 * Conventions for every call:
 *  - Return value: SSD_OK (0) or a negative ssd_status.  On error the context's
 *    state is unchanged; ssd_last_error() holds a message (thread-local).
 *  - Device pointers are plain HIP device addresses (e.g. from torch tensors);
 *    the library never allocates, frees or resizes them.
 *  - Host arrays are owned by the caller; their sizes are stated per argument.
 *  - Work is enqueued on the stream given to ssd_load.  Calls that return host
 *    data synchronise that stream before returning.
 *  - Matrices are row-major [out_features, in_features]; element type is the
 *    cfg dtype (float32, or bf16 stored as uint16 bit patterns).
 *  - One context is not thread-safe; distinct contexts are independent.
 */
#ifndef SSD_H
#define SSD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_E_ARG = -1,          /* bad argument: size, token id, pointer, cfg field */
    SSD_E_STATE = -2,        /* call not allowed in the context's current state */
    SSD_E_CAPACITY = -3,     /* the pass would write past max_ctx                */
    SSD_E_HIP = -4,          /* a HIP runtime call failed (see ssd_last_error)  */
    SSD_E_UNSUPPORTED = -5   /* e.g. non-greedy decoding                        */
} ssd_status;

/* Context states (ssd_state / ssd_check_transition). */
enum { SSD_ST_LOADED = 0, SSD_ST_READY = 1, SSD_ST_DRAFTED = 2, SSD_ST_VERIFIED = 3 };
/* Operations (ssd_check_transition). */
enum { SSD_OP_PREFILL = 0, SSD_OP_DRAFT = 1, SSD_OP_VERIFY = 2, SSD_OP_VERIFY_BLOCK = 3,
       SSD_OP_ACCEPT = 4, SSD_OP_RESET = 5 };

enum { SSD_F32 = 0, SSD_BF16 = 1 };
#define SSD_MAX_FEAT 8
#define SSD_MAX_BLOCK 32      /* largest verify block (k + 1) a context may declare */

/*
 * Model and capacity description.  Dense layers: pre-norm RMSNorm, rotary
 * embedding (rotate-half pairs (i, i+head_dim/2), base rope_theta), grouped-query
 * attention (query head h reads KV head h*n_kv_heads/n_q_heads), SwiGLU FFN,
 * untied LM head; no biases (LayerSkip summary, notation section).
 * MoE (n_experts > 0): layers >= n_dense_layers use top_k of n_experts routed
 * experts (softmax gate, not renormalised) plus n_shared shared experts, each
 * an expert_ffn-wide SwiGLU; dense layers then use dense_ffn.
 * Feature tap (n_feat > 0): each verify pass also outputs
 * fc . bf16(concat of the residual after layers feat_layers[0..n_feat))
 * (mlx-dflash README, "Architecture": context features from five layers -> fc).
 */
typedef struct {
    int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
    int32_t dtype;                 /* SSD_F32 or SSD_BF16 */
    float rms_eps, rope_theta;
    int32_t max_ctx;               /* KV capacity in positions */
    int32_t max_block;             /* largest verify block k+1 (<= SSD_MAX_BLOCK) */
    int32_t prefill_chunk;         /* rows per prefill pass (multiple of 16, <= 256) */
    int32_t n_experts, top_k, n_shared, expert_ffn, n_dense_layers, dense_ffn;
    int32_t moe_dedup;             /* 0: per-slot expert reads, 1: deduplicated */
    int32_t n_feat, feat_layers[SSD_MAX_FEAT];
} ssd_cfg;

typedef struct { const void* ptr; int64_t nbytes; } ssd_buf;

typedef struct {
    int64_t cycles;        /* draft/verify/accept cycles (or plain decode steps) */
    int64_t drafted;       /* draft tokens proposed */
    int64_t accepted;      /* draft tokens accepted */
    int64_t emitted;       /* tokens emitted by the decode loop (after prefill) */
    int64_t verify_passes; /* verify passes timed in t_verify_ms */
    double t_prefill_ms, t_draft_ms, t_verify_ms, t_accept_ms, t_decode_ms;
} ssd_stats;

/* ---- host-only helpers (no HIP call, usable without a GPU) ---------------- */

/* Checks cfg for consistency (divisibility, limits, supported dtypes).  */
ssd_status ssd_validate_cfg(const ssd_cfg* cfg);

/* Number of weight tensors ssd_load expects, and the element count of tensor i
 * in the canonical order:
 *   embed [V,d];
 *   per layer l: attn_norm [d], wq [Hq*hd,d], wk [Hkv*hd,d], wv [Hkv*hd,d],
 *     wo [d,Hq*hd], ffn_norm [d], then
 *     dense layer: w_gate [F,d], w_up [F,d], w_down [d,F]   (F = dense_ffn if MoE)
 *     MoE layer:   router [E,d], exp_gate [E,Fe,d], exp_up [E,Fe,d],
 *                  exp_down [E,d,Fe], sh_gate [S,Fe,d], sh_up [S,Fe,d], sh_down [S,d,Fe];
 *   final_norm [d], lm_head [V,d], fc [d, n_feat*d] (only when n_feat > 0).
 * Returns -1 for an invalid cfg or index. */
int32_t ssd_n_weights(const ssd_cfg* cfg);
int64_t ssd_weight_numel(const ssd_cfg* cfg, int32_t i);

/* 1 if the context reads weight tensor i after ssd_load returns, 0 if the
 * caller may free it then, -1 for an invalid cfg or index.  bf16 models copy
 * every matrix (all but embed and the norm gains) into the workspace at load,
 * in the tile order their GEMMs stream; float32 models keep every buffer. */
int32_t ssd_weight_retained(const ssd_cfg* cfg, int32_t i);

/* Device workspace size in bytes for cfg; -1 if cfg is invalid.  It holds the
 * one KV cache that draft and verify share (LayerSkip summary 4.3.3; mlx-dflash
 * README, "Apple Silicon Optimizations": the cache is kept across steps and
 * cropped on rejection, so it is allocated once at its full capacity max_ctx),
 * the activations and partial results of one pass of up to
 * max(max_block, prefill_chunk) rows, the rotary tables, the device-resident
 * block and committed-length state (mlx-dflash README, "Apple Silicon
 * Optimizations": verify ids assembled on the GPU) and, for bf16 models, the
 * packed copy of the weight matrices.  The caller allocates it (host code of
 * this library never allocates device memory). */
int64_t ssd_workspace_bytes(const ssd_cfg* cfg);

/* Skip mask of the naive layer-skip draft (MLX layer-skip blog, "Code"):
 * n_skip = max(1, round_half_even(n_layers*frac)), start = (n_layers-n_skip)/2,
 * mask[l] = 1 for l in [start, start+n_skip).  mask: host array [n_layers]. */
ssd_status ssd_skip_mask(int32_t n_layers, double frac, uint8_t* mask);

/* Draft length from measured step times (speculative decoding for MoE models,
 * abstract: a step costs its bytes over the bandwidth plus a fixed time, so
 * the best draft length follows from the fitted step times).  Under geometric
 * acceptance alpha a cycle with k drafts yields E_k = sum_{i=0..k} alpha^i
 * tokens and costs C_k = k*t_draft + t_verify[k] + t_cycle, where t_verify[k]
 * is the time of a verify pass over k+1 tokens (k = 0..kmax; k = 0 is plain
 * decoding) and t_cycle the per-cycle overhead.  *k_best = the smallest k
 * maximising E_k / C_k; *rate = that maximum (tokens per unit of time).  For
 * any cost table k_best is non-decreasing in alpha (log E_{k+1}/E_k grows with
 * alpha).  SSD_E_ARG for NULL pointers, kmax outside [0, 31], alpha outside
 * [0, 1] or a non-positive time. */
ssd_status ssd_select_k(const double* t_verify, int32_t kmax, double t_draft, double t_cycle, double alpha,
                        int32_t* k_best, double* rate);

/* Skip set as a 0/1 knapsack (MLX layer-skip blog, "Paper -> the idea": choose
 * the skipped layers to keep the draft accurate within a compute budget, with
 * hardware-measured per-layer costs and hidden-state cosine similarity as the
 * acceptance proxy).  Keeps the layer set K maximising sum_{l in K} value[l]
 * subject to sum_{l in K} cost[l] <= budget (exact dynamic programme over the
 * integer costs); mask[l] = 1 for skipped layers (host [n_layers]);
 * *kept_value = the optimum.  Costs are non-negative integers in any unit;
 * SSD_E_ARG if n_layers * (budget + 1) > 2^26, for NULL pointers or a
 * negative cost or budget. */
ssd_status ssd_knapsack_skip(const int32_t* cost, const double* value, int32_t n_layers, int64_t budget,
                             uint8_t* mask, double* kept_value);

/* State machine: next state of `op` from `state`, or SSD_E_STATE. */
ssd_status ssd_check_transition(int32_t state, int32_t op, int32_t* next_state);

const char* ssd_strerror(ssd_status s);
const char* ssd_last_error(void);

/* ---- context ----------------------------------------------------------------- */

typedef struct ssd_ctx ssd_ctx;

/* Binds one model's weights for both the draft and the verify passes: the
 * draft is the same network run on a subset of its layers, so there is one
 * weight table (LayerSkip summary 4.3.1, self-drafting with the model's own
 * early layers; MLX layer-skip blog, "Code": the draft shares the full model's
 * layer objects).  weights: device buffers, canonical order, n_weights of them,
 * sizes checked, 16-byte aligned (a zero-byte entry, such as the shared experts
 * of an MoE model with n_shared = 0, may be NULL); a device workspace of at
 * least ssd_workspace_bytes(cfg)
 * bytes, 256-byte aligned.  hip_stream: a hipStream_t (NULL = the null stream).
 * Clears the KV cache; for bf16 models packs the weight matrices into the
 * workspace (synchronously) after which the buffers ssd_weight_retained
 * reports as 0 are no longer read.  *out receives the context (free with
 * ssd_free). */
ssd_status ssd_load(const ssd_cfg* cfg, const ssd_buf* weights, int32_t n_weights,
                    ssd_buf workspace, void* hip_stream, ssd_ctx** out);
void ssd_free(ssd_ctx* ctx);

/* Back to LOADED: committed length 0, statistics cleared. */
ssd_status ssd_reset(ssd_ctx* ctx);
int32_t ssd_state(const ssd_ctx* ctx);
/* Committed KV length n (positions [0, n) hold full-model entries). */
int32_t ssd_context_length(const ssd_ctx* ctx);

/* Prefill (mlx-dflash README, "Architecture": the target's prefill fills the
 * KV cache before the decode loop; LayerSkip summary 4.3: the cache of the
 * verified tokens is what draft and verify read): runs the prompt
 * tokens[0..n) (host, ids in [0,V)) at positions 0..n-1 through all layers in
 * passes of prefill_chunk rows; *next_tok (host, may be NULL) receives argmax
 * of the last row's logits (lowest index on ties), which becomes the pending
 * token t_last at position n.  LOADED -> READY.  SSD_E_ARG for n < 1 or a
 * token outside [0, V); SSD_E_CAPACITY for n + 1 > max_ctx. */
ssd_status ssd_prefill(ssd_ctx* ctx, const int32_t* tokens, int32_t n, int32_t* next_tok);

/* Draft (LayerSkip summary 4.3.1): k tokens, each through the layers with
 * skip_mask[l] == 0 only (host array [n_layers]; NULL = no layer skipped),
 * at positions n..n+k-1, reading and writing the shared KV cache of the kept
 * layers.  drafts: host [k] or NULL.  READY -> DRAFTED.  Requires
 * 1 <= k <= max_block-1 and n+k+1 <= max_ctx. */
ssd_status ssd_draft(ssd_ctx* ctx, const uint8_t* skip_mask, int32_t k, int32_t* drafts);

/* Verify (LayerSkip summary 4.3.2; mlx-dflash "Architecture"): one pass of the
 * m block tokens [t_last, d_1..d_{m-1}] through all layers at positions
 * n..n+m-1, overwriting those KV entries.  block == NULL uses the device-
 * resident block (DRAFTED -> VERIFIED, m must be k+1); a host block [m] is
 * allowed from READY or DRAFTED (-> VERIFIED; block[0] normally t_last) and
 * replaces any drafted tokens: a harness can run the real draft passes and
 * then verify a block of known agreement with the target.
 * posterior: host [m] or NULL, receives argmax of each row's logits. */
ssd_status ssd_verify(ssd_ctx* ctx, const int32_t* block, int32_t m, int32_t* posterior);

/* Accept + rollback (mlx-dflash "Architecture" and "Apple Silicon
 * Optimizations"): a = number of leading drafts equal to the verifier's
 * predictions; emitted = d_1..d_a, p_a; the committed length becomes n+a+1 and
 * p_a becomes t_last (entries past the committed length are stale and are
 * overwritten before any read).  n_accepted, n_emitted: host scalars (may be
 * NULL); emitted: host [m] or NULL.  VERIFIED -> READY. */
ssd_status ssd_accept_rollback(ssd_ctx* ctx, int32_t* n_accepted, int32_t* emitted,
                               int32_t* n_emitted);

/* Whole decode: prefill the prompt, then loop until n_new tokens are produced
 * (the first one comes from the prefill).  skip_mask == NULL or k == 0: plain
 * greedy decode (one full pass per token, no host synchronisation per token);
 * otherwise draft/verify/accept cycles with one host synchronisation each.
 * greedy = 1: greedy decoding and greedy acceptance.  greedy = 0: sampling at
 * the temperature and seed of ssd_set_sampling (SSD_E_STATE if never set):
 * every token is drawn from softmax(logits / T) and a cycle accepts by
 * rejection sampling (LayerSkip summary 4.3.2), so the output follows the full
 * model's sampling distribution; exit-state reuse is not used.  Other values
 * -> SSD_E_UNSUPPORTED.  out: host [n_new]; stats: host or NULL.  Leaves the
 * context READY. */
/* Sampling parameters of ssd_generate(greedy = 0): temperature T > 0 and the
 * seed of the Philox4x64-10 stream (key (seed, 0), counter (cycle, slot,
 * purpose, 0): purposes 0 draft token of slot j, 1 accept test of draft i,
 * 2 final token of a cycle that accepted a drafts; u = top 24 bits / 2^24).
 * A draft d_i ~ q_i is accepted when u * q_i(d_i) < p_{i-1}(d_i); the first
 * rejection draws from max(0, p - q) normalised, a full accept from p_k.  A
 * draw takes the smallest index whose running sum of weights exceeds u times
 * their total.  SSD_E_ARG for T <= 0 or not finite. */
ssd_status ssd_set_sampling(ssd_ctx* ctx, float temperature, uint64_t seed);

ssd_status ssd_generate(ssd_ctx* ctx, const int32_t* prompt, int32_t n_prompt, int32_t n_new,
                        int32_t greedy, const uint8_t* skip_mask, int32_t k,
                        int32_t* out, ssd_stats* stats);

/* Options: SSD_OPT_GRAPHS (default 1) replays each decode-loop pass (draft
 * step, verify, plain decode step) as a HIP graph captured on first use;
 * 0 launches every kernel directly.  Both give bitwise-identical results.
 * hip_stream must not be the null stream while graphs are on.
 * SSD_OPT_MOE_DEDUP switches an MoE model between per-slot (0) and
 * deduplicated (1) expert reads (speculative decoding for MoE models,
 * abstract); outputs are bitwise identical.
 * SSD_OPT_TRACE (default 0): decode-loop passes also record the float32
 * residual after every layer (ssd_read_trace); a test hook. */
/* SSD_OPT_KVQ (default 0): when a draft's mask is a tail {E..L-1} (the
 * LayerSkip early-exit draft, 1 <= E < L), the draft saves each row's residual
 * after layer E-1 and the verify of that draft runs the last drafted token
 * through layers 0..E-1, then all rows through layers E..L-1 only, reusing
 * the draft's KV entries of layers < E (LayerSkip summary 4.3.3, the exit
 * query cache, read as the residual entering layer E).  Posterior and logits
 * equal the full verify's bit for bit.  The feature tap is not recomputed by
 * such a verify.  Other masks, and host blocks, verify in full. */
/* SSD_OPT_TILE_GROUPS (default 0 = 512): passes wider than 32 rows run the
 * layer GEMMs on workgroups of 64 rows x 4 * ntw column tiles, ntw = 4, 2 or
 * 1 (gate/up: 2 or 1), the widest that leaves at least this many
 * workgroups.  The grouping never changes a result; a test and measurement
 * hook (a small value forces the widest grouping).  value >= 0. */
enum { SSD_OPT_GRAPHS = 0, SSD_OPT_MOE_DEDUP = 1, SSD_OPT_TRACE = 2, SSD_OPT_KVQ = 3, SSD_OPT_TILE_GROUPS = 4 };
ssd_status ssd_set_option(ssd_ctx* ctx, int32_t option, int32_t value);

/* Statistics accumulated since load/reset (per-phase times from HIP events). */
ssd_status ssd_get_stats(const ssd_ctx* ctx, ssd_stats* stats);

/* ---- test and measurement hooks -------------------------------------------------- */

/* Logits (float32) of the last pass: host [rows * V], rows <= rows of that pass
 * (prefill keeps only its last row). */
ssd_status ssd_read_logits(ssd_ctx* ctx, float* host, int32_t rows);
/* Residual after every layer of the last decode-loop pass (SSD_OPT_TRACE on):
 * host [n_layers * rows * d] float32, layer-major. */
ssd_status ssd_read_trace(ssd_ctx* ctx, float* host, int32_t rows);
/* Stored operands of one layer of the last decode-loop pass (SSD_OPT_TRACE on;
 * rows <= min(rows of that pass, max_block)), the values later kernels read:
 * point 0 the QKV GEMM input (bf16(x * attn_norm) for bf16 models, the normed
 * row for float32 models) [rows][d], 1 q after the rotary embedding
 * [rows][n_q_heads * head_dim], 2 the attention output [rows][n_q_heads *
 * head_dim], 3 the residual after the attention block, float32 [rows][d],
 * 4 the gate/up GEMM input [rows][d] (bf16(x * ffn_norm) for bf16 models,
 * also the row the MoE router and experts share), 5 the SwiGLU activation [rows][F] (MoE layers: [rows]
 * [top_k + n_shared][expert_ffn], routed slots then shared experts); cfg
 * dtype except point 3.  layer == n_layers with
 * point 0: the LM head's input of rows [0, rows).  Layers a draft skipped keep
 * an earlier pass's values.  host: caller-owned, rows x the row size. */
ssd_status ssd_read_trace_point(ssd_ctx* ctx, int32_t layer, int32_t point, int32_t rows, void* host);
/* Acceptance proxy of every layer from the last decode-loop pass (SSD_OPT_TRACE
 * on; the pass must have run every layer): cos[l] = mean over its first rows
 * rows of cos(input of layer l, output of layer l), the input of layer 0
 * being the token embedding; computed in double on the host.  A layer that
 * barely turns the residual (cos near 1) is a good one to skip. */
ssd_status ssd_layer_cosines(ssd_ctx* ctx, int32_t rows, double* cos);
/* KV cache entries of one layer, positions [pos0, pos0+n): host k and v,
 * each [n_kv_heads * n * head_dim] in the cfg dtype (bf16 bits or float32). */
ssd_status ssd_read_kv(ssd_ctx* ctx, int32_t layer, int32_t pos0, int32_t n, void* k_host, void* v_host);
/* Feature-tap output of the last verify pass: host [rows * d] bf16 bits. */
ssd_status ssd_read_features(ssd_ctx* ctx, uint16_t* host, int32_t rows);
/* Injects expert ids for the next passes: host [n_layers][n][top_k] (entries for
 * dense layers ignored); n == 0 returns to the router's own choice.  Passes
 * are then limited to n rows (SSD_E_ARG otherwise).  Switching between
 * injected and router-chosen ids drops the captured pass graphs (they are
 * captured again on next use); the injected ids are read at every replay. */
ssd_status ssd_set_routing(ssd_ctx* ctx, const int32_t* ids, int32_t n);
/* Routed-expert union size per layer of the last MoE pass: host [n_layers]. */
ssd_status ssd_read_union(ssd_ctx* ctx, int32_t* host);
/* Runs the accept kernel on host drafts d[k] and predictions p[k+1];
 * *a receives the accepted length.  Does not change the context's state. */
ssd_status ssd_test_accept(ssd_ctx* ctx, const int32_t* d, const int32_t* p, int32_t k, int32_t* a);
/* Allocation-free form of ssd_test_accept, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  No context: the accept kernel's staging (block and
 * predictions), its counters and its outputs live in a static device array of
 * SSD_NOALLOC_SCRATCH_BYTES per GPU, which each GPU keeps until the process
 * ends; its address is looked up once per device, on the first call made with
 * that device current.  Same inputs and result as ssd_test_accept: d[k] and
 * p[k+1] host arrays, *a = accepted length; SSD_E_ARG for k outside
 * [0, SSD_MAX_BLOCK - 1] or NULL pointers.  Runs on hip_stream (NULL = the
 * null stream) and synchronises it.  Calls no allocator.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (other threads or
 * streams) race. */
#define SSD_NOALLOC_SCRATCH_BYTES 1024
ssd_status ssd_test_accept_noalloc(const int32_t* d, const int32_t* p, int32_t k, void* hip_stream, int32_t* a);
/* Test hook: `trials` sampled cycles on host logits with the decode loop's
 * sampling kernels, cycle numbers cycle0, cycle0 + 1, ... (cycle0 + trials
 * <= 2^31 - 1, else SSD_E_ARG); each cycle draws its k drafts from the draft
 * rows, then accepts.  target [(k+1) * V] rows p_0..p_k, draft [k * V] (row
 * i-1 is q for draft i), float32, V <= vocab, k + 1 <= max_block.  out: host
 * [trials * (k+2)]: a, the a+1 emitted tokens, -1 padding.  Overwrites the
 * context's logits (read_logits); the decode state is not touched. */
ssd_status ssd_test_spec_cycle(ssd_ctx* ctx, const float* target, const float* draft, int32_t k, int32_t V,
                               float temperature, uint64_t seed, uint64_t cycle0, int32_t trials, int32_t* out);
/* Times `iters` back-to-back launches of one layer operation at m rows on the
 * context's stream with HIP events; *avg_us receives the mean duration.
 * op: 0 = gate/up GEMM (+SwiGLU), 1 = down GEMM, 2 = qkv GEMM (+RoPE/KV),
 *     3 = o GEMM, 4 = lm_head GEMM, 5 = attention, 6 = MoE expert FFN
 *     (router, grouping, expert GEMMs, combine), 7 = streaming read of the LM
 *     head matrix with 256*m workgroups (achievable HBM read bandwidth),
 *     8 = plain float32 copy of m MiB (capped by the buffers) from the LM head
 *     matrix into scratch (a known-size read + write for counter calibration).
 * Launch i uses the weights of the i-th layer (cyclically, starting at
 * `layer`, among layers of the same kind), so consecutive launches stream
 * different weights as a real pass does.  Writes only scratch activations and
 * KV entries past the committed length. */
ssd_status ssd_time_op(ssd_ctx* ctx, int32_t op, int32_t layer, int32_t m, int32_t iters,
                       float* avg_us);

#ifdef __cplusplus
}
#endif
#endif /* SSD_H */
