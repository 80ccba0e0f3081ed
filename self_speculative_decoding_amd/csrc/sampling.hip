// Speculative sampling on gfx950: the non-greedy draft and accept.
//
// LayerSkip summary 4.3.2 (self-verification): under sampling, rejection
// sampling keeps the output distribution equal to the full model's, following
// the standard speculative decoding protocol.  Per cycle with k drafts:
// d_i ~ q_i (the draft's softmax(logits / T)); d_i is accepted with
// probability min(1, p_{i-1}(d_i) / q_i(d_i)) in order; the first rejection
// emits a token drawn from max(0, p_{i-1} - q_i) normalised and ends the
// cycle; if all k pass, a token is drawn from p_k.  Plain sampled decoding is
// the k = 0 cycle.
//
// Random numbers: Philox4x64-10 (Salmon et al., "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011) with key (seed, 0) and counter (cycle, slot,
// purpose, 0); the first output word's top 24 bits give u in [0, 1), exact in
// float.  Purposes: 0 draft of slot j, 1 accept test of draft i, 2 the final
// token of a cycle that accepted a drafts (slot a).  The cycle counter lives
// in device memory (state[2]), so nothing on the host has to follow it.
//
// A draw from weights w takes the smallest j whose running sum exceeds u
// times the total.  Rows are split into chunks of SMP_CH columns and every
// step is three launches, each reading its rows coalesced and reducing in a
// fixed order:
//   stats: per (row, chunk) the chunk max m and the sum of exp((l - m) / T);
//   sums:  every workgroup combines the row stats (same code, same order, so
//          all agree), takes the cycle's accept decisions and sums the final
//          distribution's weights over its chunk; workgroup 0 publishes the
//          decisions;
//   pick:  one workgroup finds the chunk holding u times the total, scans it
//          and commits the tokens.
#include "device.h"

namespace ssd {

constexpr int SMP_T = 256;                   // threads of every sampling workgroup
constexpr int SMP_PER = 8;                   // columns per thread in a chunk
constexpr int SMP_CH = SMP_T * SMP_PER;      // columns per chunk
constexpr int SMP_MAXB = 32;                 // largest block (k + 1) of a cycle
constexpr int SMP_MAXROWS = 2 * SMP_MAXB - 1;
constexpr int SMP_MAXCH = 128;               // chunks of the widest row (vocabulary <= 262144)
static_assert(SMP_CH == SMP_CHUNK && SMP_MAXROWS == SMP_ROWS, "scratch layout");

enum { SMP_DRAFT = 0, SMP_CYCLE = 1, SMP_FIRST = 2 };

// the final draw of a step, decided by the sums kernel
struct SmpCtl {
  int a;                   // accepted drafts
  int resid;               // 1: draw from max(0, p - q) of rows (rp, rq); 0: from row rp
  int rp, rq;
  float Mp, rZp, Mq, rZq;  // row max and 1 / sum of exp((l - max) / T)
  float u;                 // uniform of the final draw
};
static_assert(sizeof(SmpCtl) <= SMP_CTL_BYTES, "scratch layout");

// target rows tl[0..nt), then draft rows dl[0..)
struct RowSrc {
  const float* tl;
  const float* dl;
  int ld, nt;
  __device__ __forceinline__ const float* row(int r) const {
    return r < nt ? tl + (size_t)r * ld : dl + (size_t)(r - nt) * ld;
  }
};

__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                                 uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(0xD2E7470EE14C6C93ull, c0), lo0 = 0xD2E7470EE14C6C93ull * c0;
    const uint64_t hi1 = __umul64hi(0xCA5A826395121157ull, c2), lo1 = 0xCA5A826395121157ull * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B97F4A7C15ull;
    k1 += 0xBB67AE8584CAA73Bull;
  }
  return c0;
}

__device__ __forceinline__ float uniform24(uint64_t seed, uint64_t cycle, uint64_t slot, uint64_t purpose) {
  return (float)(philox_word0(cycle, slot, purpose, 0, seed, 0) >> 40) * (1.0f / 16777216.0f);
}

// fixed-order workgroup reduction: wave butterfly, then the wave values in order
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = MAX ? fmaxf(v, w) : v + w;
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < SMP_T / 64; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

// Weight of column j in the final distribution; the sums and pick kernels
// evaluate it with this one expression (products rounded separately, no
// contraction), so both see the same value.  plain: exp((p_j - Mp) / T);
// residual: max(0, p_j / Zp - q_j / Zq).  *plain: exp((p_j - Mp) / T).
__device__ __forceinline__ float smp_weight(const SmpCtl& c, const float* p, const float* q, int j, float invT,
                                            float* plain) {
  const float ep = expf((p[j] - c.Mp) * invT);
  *plain = ep;
  if (!c.resid) return ep;
  const float eq = expf((q[j] - c.Mq) * invT);
  return fmaxf(__fmul_rn(ep, c.rZp) - __fmul_rn(eq, c.rZq), 0.f);
}

// grid (chunks, rows): stats[r * nch + c] = (m, sum exp((l - m) / T)) over the
// chunk's columns; keep (or null) receives a copy of row 0.
__global__ __launch_bounds__(SMP_T) void smp_stats_kernel(RowSrc src, int V, float invT, float2* stats, int nch,
                                                          float* keep) {
  __shared__ float red[SMP_T / 64];
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const float* x = src.row(r);
  float v[SMP_PER];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = c * SMP_CH + i * SMP_T + tid;
    v[i] = j < V ? x[j] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  if (keep != nullptr && r == 0) {
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) {
      const int j = c * SMP_CH + i * SMP_T + tid;
      if (j < V) keep[j] = v[i];
    }
  }
  m = block_reduce<true>(m, red);
  float s = 0.f;
  if (m > -INFINITY) {
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) s += expf((v[i] - m) * invT);
  }
  s = block_reduce<false>(s, red);
  if (tid == 0) stats[(size_t)r * nch + c] = make_float2(m, s);
}

// grid (chunks): row summaries, the step's decisions, and the chunk sums of
// the final distribution's weights (csum[c]) and of exp((p_rp - Mp) / T)
// (csum[nch + c], the fallback when a residual has no mass).
//   SMP_DRAFT: one row (the draft pass's logits), u(cycle, slot, 0).
//   SMP_CYCLE: rows p_0..p_k then q_1..q_k, drafts block[1..k], cycle state[2].
//   SMP_FIRST: the k = 0 cycle numbered 0.
__global__ __launch_bounds__(SMP_T) void smp_sums_kernel(int mode, RowSrc src, int V, int k, float invT,
                                                         uint64_t seed, const float2* stats, int nch,
                                                         const int* state, const int* block, int slot, float* csum,
                                                         SmpCtl* ctl) {
  __shared__ float red[SMP_T / 64];
  __shared__ float sM[SMP_MAXROWS], sZ[SMP_MAXROWS];
  __shared__ float sp_d[SMP_MAXB], sq_d[SMP_MAXB];
  __shared__ SmpCtl sc;
  const int tid = threadIdx.x;
  const int nrows = 2 * k + 1;
  if (mode != SMP_DRAFT && tid >= 1 && tid <= k) {   // the drafts' logits, fetched in parallel
    const int tok = min(max(block[tid], 0), V - 1);
    sp_d[tid] = src.row(tid - 1)[tok];
    sq_d[tid] = src.row(k + tid)[tok];
  }
  // row summaries: 16 lanes per row, lane l takes chunks l, l + 16, ...;
  // fixed butterflies, so every workgroup gets the same M and Z
  {
    const int g = tid >> 4, l = tid & 15;
    for (int r0 = 0; r0 < nrows; r0 += SMP_T / 16) {
      const int r = r0 + g;
      const float2* st = stats + (size_t)min(r, nrows - 1) * nch;
      float M = -INFINITY;
#pragma unroll 4
      for (int c = l; c < nch; c += 16) M = fmaxf(M, st[c].x);
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
      float Z = 0.f;
#pragma unroll 4
      for (int c = l; c < nch; c += 16) Z += st[c].y * expf((st[c].x - M) * invT);
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) Z += __shfl_xor(Z, o);
      if (r < nrows && l == 0) {
        sM[r] = M;
        sZ[r] = Z;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const uint64_t cycle = mode == SMP_FIRST ? 0 : (uint64_t)state[2];
    SmpCtl d;
    d.resid = 0;
    d.rq = 0;
    d.Mq = 0.f;
    d.rZq = 0.f;
    if (mode == SMP_DRAFT) {
      d.a = 0;
      d.rp = 0;
      d.u = uniform24(seed, cycle, slot, 0);
    } else {
      int a = k;
      for (int i = 1; i <= k; ++i) {
        const int rp = i - 1, rq = k + i;
        const float pd = expf((sp_d[i] - sM[rp]) * invT) / sZ[rp];
        const float qd = expf((sq_d[i] - sM[rq]) * invT) / sZ[rq];
        if (uniform24(seed, cycle, i, 1) * qd < pd) continue;
        a = i - 1;
        d.resid = 1;
        d.rq = rq;
        d.Mq = sM[rq];
        d.rZq = 1.0f / sZ[rq];
        break;
      }
      d.a = a;
      d.rp = d.resid ? a : k;
      d.u = uniform24(seed, cycle, a, 2);
    }
    d.Mp = sM[d.rp];
    d.rZp = 1.0f / sZ[d.rp];
    sc = d;
  }
  __syncthreads();
  const SmpCtl d = sc;
  const float* p = src.row(d.rp);
  const float* q = src.row(d.rq);
  float s = 0.f, sp = 0.f;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int j = blockIdx.x * SMP_CH + i * SMP_T + tid;
    if (j < V) {
      float e;
      s += smp_weight(d, p, q, j, invT, &e);
      sp += e;
    }
  }
  s = block_reduce<false>(s, red);
  sp = block_reduce<false>(sp, red);
  if (tid == 0) {
    csum[blockIdx.x] = s;
    csum[nch + blockIdx.x] = sp;
    if (blockIdx.x == 0) *ctl = d;
  }
}

// One workgroup: the draw, then the commit.
//   SMP_DRAFT: block[slot + 1] = token.
//   SMP_CYCLE: the emitted d_1..d_a + token go to result[2..] and
//     outlog[state[1]..] (outlog may be null), result[0..1] = a, a+1; the
//     committed and emitted counts advance by a+1, block[0] = token, the
//     cycle counter by one; trial_out (or null) gets a, the emitted tokens
//     and -1 up to k+2 entries.
//   SMP_FIRST: the token replaces the prefill's argmax in block[0] and the
//     log; the cycle counter becomes 1.
__global__ __launch_bounds__(SMP_T) void smp_pick_kernel(int mode, RowSrc src, int V, int k, int slot, float invT,
                                                         const float* csum, int nch, const SmpCtl* ctl, int* block,
                                                         int* state, int* outlog, int* result, int* trial_out) {
  __shared__ float red[SMP_T / 64];
  __shared__ float scan[SMP_T / 64];
  __shared__ float scs[2 * SMP_MAXCH];
  __shared__ SmpCtl sc;
  __shared__ int s_chunk, s_pick;
  __shared__ float s_target;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int c = tid; c < 2 * nch; c += SMP_T) scs[c] = csum[c];
  __syncthreads();
  if (tid == 0) {
    SmpCtl d = *ctl;
    const float* cs = scs;
    float total = 0.f;
    for (int c = 0; c < nch; ++c) total += cs[c];
    if (d.resid && !(total > 0.f)) {   // no residual mass: draw from p itself
      d.resid = 0;
      cs = scs + nch;
      total = 0.f;
      for (int c = 0; c < nch; ++c) total += cs[c];
    }
    const float target = d.u * total;
    int chunk = -1, last = nch - 1;
    float run = 0.f, before = 0.f;
    for (int c = 0; c < nch; ++c) {
      if (cs[c] > 0.f) last = c;
      if (chunk < 0) {
        before = run;
        run += cs[c];
        if (run > target) chunk = c;
      }
    }
    if (chunk < 0) {   // rounding left the target uncovered: the last positive column
      chunk = last;
      s_target = INFINITY;
    } else {
      s_target = target - before;
    }
    s_chunk = chunk;
    s_pick = -1;
    sc = d;
  }
  __syncthreads();
  const SmpCtl d = sc;
  const float* p = src.row(d.rp);
  const float* q = src.row(d.rq);
  // thread t owns the chunk's columns [8t, 8t + 8), scanned in order
  const int j0 = min(s_chunk * SMP_CH + tid * SMP_PER, V), j1 = min(j0 + SMP_PER, V);
  float w[SMP_PER];
  float S = 0.f;
  int lastpos = -1;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    float e;
    w[i] = j0 + i < j1 ? smp_weight(d, p, q, j0 + i, invT, &e) : 0.f;
    S += w[i];
    if (w[i] > 0.f) lastpos = j0 + i;
  }
  float incl = S;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.f;
  if (lane == 63) scan[wave] = incl;
  __syncthreads();
  float off = 0.f;
  for (int v = 0; v < wave; ++v) off += scan[v];
  // start of thread t == end of thread t-1 bit for bit, so at most one owner
  const float start = off + excl, end = off + incl;
  const float target = s_target;
  if (S > 0.f && start <= target && target < end) {
    float acc = start;
    int pick = lastpos;
#pragma unroll
    for (int i = 0; i < SMP_PER; ++i) {
      acc += w[i];
      if (acc > target && w[i] > 0.f) {
        pick = j0 + i;
        break;
      }
    }
    s_pick = pick;
  }
  const int lp = (int)block_reduce<true>((float)lastpos, red);   // its barrier also orders the pick write
  const int pk = s_pick;
  const int tok = pk >= 0 ? pk : (lp >= 0 ? lp : min(s_chunk * SMP_CH, V - 1));
  if (mode == SMP_DRAFT) {
    if (tid == 0) block[slot + 1] = tok;
    return;
  }
  if (mode == SMP_FIRST) {
    if (tid == 0) {
      block[0] = tok;
      outlog[state[1] - 1] = tok;
      state[2] = 1;
    }
    return;
  }
  const int a = d.a;
  const int base = state[1];
  if (tid <= a) {
    const int t = tid < a ? block[tid + 1] : tok;
    result[2 + tid] = t;
    if (outlog != nullptr) outlog[base + tid] = t;
  }
  if (trial_out != nullptr && tid < k + 2)
    trial_out[tid] = tid == 0 ? a : (tid - 1 < a ? block[tid] : (tid - 1 == a ? tok : -1));
  __syncthreads();   // every thread has read state[1] and block[1..a]
  if (tid == 0) {
    result[0] = a;
    result[1] = a + 1;
    state[0] += a + 1;
    state[1] += a + 1;
    state[2] += 1;
    block[0] = tok;
  }
}

static hipError_t smp_run(int mode, RowSrc src, int nrows, int V, int k, int slot, float T, uint64_t seed,
                          int* block, int* state, int* outlog, int* result, int* trial_out, float* keep,
                          const SmpBufs& b, hipStream_t s) {
  const int nch = (V + SMP_CH - 1) / SMP_CH;
  if (k < 0 || k + 1 > SMP_MAXB || V < 1 || src.ld < V || nch > b.nch_max || nch > SMP_MAXCH || !(T > 0.f))
    return hipErrorInvalidValue;
  const float invT = 1.0f / T;
  float2* stats = (float2*)b.stats;
  SmpCtl* ctl = (SmpCtl*)b.ctl;
  smp_stats_kernel<<<dim3(nch, nrows), SMP_T, 0, s>>>(src, V, invT, stats, nch, keep);
  smp_sums_kernel<<<nch, SMP_T, 0, s>>>(mode, src, V, k, invT, seed, stats, nch, state, block, slot, b.csum, ctl);
  smp_pick_kernel<<<1, SMP_T, 0, s>>>(mode, src, V, k, slot, invT, b.csum, nch, ctl, block, state, outlog, result,
                                      trial_out);
  return hipGetLastError();
}

hipError_t launch_spec_accept(const float* tl, const float* dl, int ld, int V, int k, float T, uint64_t seed,
                              int* block, int* state, int* outlog, int* result, int* trial_out, const SmpBufs& b,
                              hipStream_t s) {
  return smp_run(SMP_CYCLE, RowSrc{tl, dl, ld, k + 1}, 2 * k + 1, V, k, 0, T, seed, block, state, outlog, result,
                 trial_out, nullptr, b, s);
}

hipError_t launch_draft_sample(const float* l, int V, float T, uint64_t seed, int* block, const int* state, int slot,
                               float* keep, const SmpBufs& b, hipStream_t s) {
  if (slot < 0 || slot + 2 > SMP_MAXB) return hipErrorInvalidValue;
  return smp_run(SMP_DRAFT, RowSrc{l, l, V, 1}, 1, V, 0, slot, T, seed, block, (int*)state, nullptr, nullptr,
                 nullptr, keep, b, s);
}

hipError_t launch_first_sample(const float* l, int V, float T, uint64_t seed, int* block, int* state, int* outlog,
                               const SmpBufs& b, hipStream_t s) {
  return smp_run(SMP_FIRST, RowSrc{l, l, V, 1}, 1, V, 0, 0, T, seed, block, state, outlog, nullptr, nullptr,
                 nullptr, b, s);
}

}  // namespace ssd
