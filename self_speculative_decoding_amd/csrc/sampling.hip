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
// times the total.  Everything runs in one 1024-thread workgroup per row or
// per cycle, with reductions and scans in a fixed order.
#include "device.h"

namespace ssd {

constexpr int SMP_T = 1024;    // threads of every sampling workgroup
constexpr int SMP_MAXB = 32;   // largest block (k + 1) of a cycle

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

struct SmpShared {
  float red[SMP_T / 64];
  float scan[SMP_T / 64];
  int pick;
  int drafts[SMP_MAXB];
};

// fixed-order block reduction: wave butterfly, then the 16 wave values in order
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, SmpShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = MAX ? fmaxf(v, w) : v + w;
  }
  if (lane == 0) sh.red[wave] = v;
  __syncthreads();
  float r = sh.red[0];
#pragma unroll
  for (int w = 1; w < SMP_T / 64; ++w) r = MAX ? fmaxf(r, sh.red[w]) : r + sh.red[w];
  __syncthreads();
  return r;
}

// max and sum of exp((l - max) / T) of one row of V logits
__device__ __forceinline__ void row_stats(const float* l, int V, float invT, SmpShared& sh, float& M, float& Z) {
  float m = -INFINITY;
  for (int j = threadIdx.x; j < V; j += SMP_T) m = fmaxf(m, l[j]);
  M = block_reduce<true>(m, sh);
  float z = 0.f;
  for (int j = threadIdx.x; j < V; j += SMP_T) z += expf((l[j] - M) * invT);
  Z = block_reduce<false>(z, sh);
}

// Draw from weights w(0..V-1) with u: thread t owns the contiguous chunk
// [t*C, t*C + C); chunk sums are scanned in a fixed order, the thread whose
// range holds u * total walks its chunk.  Falls back to the last index with a
// positive weight when rounding leaves the target uncovered.
template <typename W>
__device__ int draw_block(W w, int V, float u, SmpShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = (V + SMP_T - 1) / SMP_T;
  const int j0 = min(tid * C, V), j1 = min(j0 + C, V);
  float S = 0.f;
  int lastpos = -1;
  for (int j = j0; j < j1; ++j) {
    const float x = w(j);
    S += x;
    if (x > 0.f) lastpos = j;
  }
  float incl = S;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.f;
  if (lane == 63) sh.scan[wave] = incl;
  if (tid == 0) sh.pick = -1;
  __syncthreads();
  float off = 0.f, total = 0.f;
  for (int v = 0; v < SMP_T / 64; ++v) {
    if (v < wave) off += sh.scan[v];
    total += sh.scan[v];
  }
  const float start = off + excl, end = off + incl;
  const float target = u * total;
  if (S > 0.f && start <= target && target < end) {
    float acc = start;
    int pick = lastpos;
    for (int j = j0; j < j1; ++j) {
      acc += w(j);
      if (acc > target) {
        pick = j;
        break;
      }
    }
    sh.pick = pick;
  }
  const int lp = (int)block_reduce<true>((float)lastpos, sh);   // also orders the pick write
  const int p = sh.pick;
  __syncthreads();
  return p >= 0 ? p : (lp >= 0 ? lp : 0);
}

// One draft/verify/accept cycle of speculative sampling.  tl: target rows
// p_0..p_k, dl: draft rows (row i-1 is q for draft i), both ld floats apart.
// drafts (when !sample_drafts): the k draft tokens.  Leaves the accepted count
// in *a_out and the emitted tokens d_1..d_a, final in sh.drafts[0..a].
__device__ void spec_cycle(const float* tl, const float* dl, int ld, int V, int k, float invT, uint64_t seed,
                           uint64_t cycle, const int* drafts, bool sample_drafts, SmpShared& sh, int* a_out) {
  float M, Z;
  if (sample_drafts) {
    for (int i = 0; i < k; ++i) {
      const float* q = dl + (size_t)i * ld;
      row_stats(q, V, invT, sh, M, Z);
      const float u = uniform24(seed, cycle, i, 0);
      const int d = draw_block([&](int j) { return expf((q[j] - M) * invT); }, V, u, sh);
      if (threadIdx.x == 0) sh.drafts[i] = d;
    }
  } else if (threadIdx.x < k) {
    sh.drafts[threadIdx.x] = drafts[threadIdx.x];
  }
  __syncthreads();
  int a = k;
  int fin = -1;
  for (int i = 1; i <= k; ++i) {
    const float* p = tl + (size_t)(i - 1) * ld;
    const float* q = dl + (size_t)(i - 1) * ld;
    float Mp, Zp, Mq, Zq;
    row_stats(p, V, invT, sh, Mp, Zp);
    row_stats(q, V, invT, sh, Mq, Zq);
    const int d = sh.drafts[i - 1];
    const float pd = expf((p[d] - Mp) * invT) / Zp, qd = expf((q[d] - Mq) * invT) / Zq;
    const float u = uniform24(seed, cycle, i, 1);
    if (u * qd < pd) continue;
    a = i - 1;
    const float rp = 1.0f / Zp, rq = 1.0f / Zq;
    const float ur = uniform24(seed, cycle, i - 1, 2);
    fin = draw_block([&](int j) { return fmaxf(expf((p[j] - Mp) * invT) * rp - expf((q[j] - Mq) * invT) * rq, 0.f); },
                     V, ur, sh);
    break;
  }
  if (a == k) {
    const float* p = tl + (size_t)k * ld;
    row_stats(p, V, invT, sh, M, Z);
    fin = draw_block([&](int j) { return expf((p[j] - M) * invT); }, V, uniform24(seed, cycle, k, 2), sh);
  }
  __syncthreads();
  if (threadIdx.x == 0) sh.drafts[a] = fin;
  __syncthreads();
  *a_out = a;
}

// Decode-loop cycle: drafts are block[1..k]; commits like the greedy accept
// (emitted tokens to result[2..] and the log, committed and emitted counts
// advance by a+1, the final token becomes t_last) and advances the cycle.
__global__ __launch_bounds__(SMP_T) void spec_accept_kernel(const float* tl, const float* dl, int ld, int V, int k,
                                                            float invT, uint64_t seed, int* block, int* state,
                                                            int* outlog, int* result) {
  __shared__ SmpShared sh;
  int a;
  spec_cycle(tl, dl, ld, V, k, invT, seed, (uint64_t)state[2], block + 1, false, sh, &a);
  const int base = state[1];
  __syncthreads();
  if (threadIdx.x <= a) {
    const int tok = sh.drafts[threadIdx.x];
    result[2 + threadIdx.x] = tok;
    outlog[base + threadIdx.x] = tok;
  }
  if (threadIdx.x == 0) {
    result[0] = a;
    result[1] = a + 1;
    state[0] += a + 1;
    state[1] += a + 1;
    state[2] += 1;
    block[0] = sh.drafts[a];
  }
}

// Test cycles: workgroup t runs cycle cycle0 + t with drafts drawn from the
// draft rows; out[t*(k+2)]: a, then the a+1 emitted tokens, then -1.
__global__ __launch_bounds__(SMP_T) void spec_test_kernel(const float* tl, const float* dl, int ld, int V, int k,
                                                          float invT, uint64_t seed, uint64_t cycle0, int* out) {
  __shared__ SmpShared sh;
  int a;
  spec_cycle(tl, dl, ld, V, k, invT, seed, cycle0 + blockIdx.x, nullptr, true, sh, &a);
  int* o = out + (size_t)blockIdx.x * (k + 2);
  if (threadIdx.x == 0) o[0] = a;
  if (threadIdx.x < k + 1) o[1 + threadIdx.x] = threadIdx.x <= a ? sh.drafts[threadIdx.x] : -1;
}

// Draft step `slot` of a sampled cycle: draws d_{slot+1} from the pass's
// logits row with u(cycle, slot, 0), and keeps the row for the accept.
__global__ __launch_bounds__(SMP_T) void draft_sample_kernel(const float* l, int V, float invT, uint64_t seed,
                                                             const int* state, int slot, int* tok, float* keep) {
  __shared__ SmpShared sh;
  for (int j = threadIdx.x; j < V; j += SMP_T) keep[j] = l[j];
  float M, Z;
  row_stats(l, V, invT, sh, M, Z);
  const int d = draw_block([&](int j) { return expf((l[j] - M) * invT); }, V,
                           uniform24(seed, (uint64_t)state[2], slot, 0), sh);
  if (threadIdx.x == 0) *tok = d;
}

// First token after a sampled prefill: drawn from the prefill's last-row
// logits as cycle 0's final token (slot 0); the cycle counter becomes 1.
__global__ __launch_bounds__(SMP_T) void first_sample_kernel(const float* l, int V, float invT, uint64_t seed,
                                                             int* block, int* state, int* outlog) {
  __shared__ SmpShared sh;
  float M, Z;
  row_stats(l, V, invT, sh, M, Z);
  const int d = draw_block([&](int j) { return expf((l[j] - M) * invT); }, V, uniform24(seed, 0, 0, 2), sh);
  if (threadIdx.x == 0) {
    block[0] = d;
    outlog[state[1] - 1] = d;
    state[2] = 1;
  }
}

hipError_t launch_spec_accept(const float* tl, const float* dl, int ld, int V, int k, float T, uint64_t seed,
                              int* block, int* state, int* outlog, int* result, hipStream_t s) {
  if (k < 0 || k + 1 > SMP_MAXB || V < 1 || ld < V || !(T > 0.f)) return hipErrorInvalidValue;
  spec_accept_kernel<<<1, SMP_T, 0, s>>>(tl, dl, ld, V, k, 1.0f / T, seed, block, state, outlog, result);
  return hipGetLastError();
}

hipError_t launch_spec_test(const float* tl, const float* dl, int ld, int V, int k, float T, uint64_t seed,
                            uint64_t cycle0, int trials, int* out, hipStream_t s) {
  if (k < 0 || k + 1 > SMP_MAXB || V < 1 || ld < V || trials < 1 || !(T > 0.f)) return hipErrorInvalidValue;
  spec_test_kernel<<<trials, SMP_T, 0, s>>>(tl, dl, ld, V, k, 1.0f / T, seed, cycle0, out);
  return hipGetLastError();
}

hipError_t launch_draft_sample(const float* l, int V, float T, uint64_t seed, const int* state, int slot, int* tok,
                               float* keep, hipStream_t s) {
  if (V < 1 || slot < 0 || !(T > 0.f)) return hipErrorInvalidValue;
  draft_sample_kernel<<<1, SMP_T, 0, s>>>(l, V, 1.0f / T, seed, state, slot, tok, keep);
  return hipGetLastError();
}

hipError_t launch_first_sample(const float* l, int V, float T, uint64_t seed, int* block, int* state, int* outlog,
                               hipStream_t s) {
  if (V < 1 || !(T > 0.f)) return hipErrorInvalidValue;
  first_sample_kernel<<<1, SMP_T, 0, s>>>(l, V, 1.0f / T, seed, block, state, outlog);
  return hipGetLastError();
}

}  // namespace ssd
