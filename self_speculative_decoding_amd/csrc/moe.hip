// Routed-expert FFN of an MoE verify pass on gfx950 (bf16).
//
// A pass of M tokens picks top_k of E routed experts per token (router
// softmax, lowest index on ties, gate = the softmax probability, not
// renormalised) and adds n_shared shared experts; every expert is a SwiGLU of
// width fe.  The expert reads come in the two forms the speculative decoding
// for MoE models abstract compares:
//   per-slot: every (token, slot) pair streams its expert's weights itself;
//   dedup:    the pairs are grouped by expert (count, prefix sum, scatter, all
//             integer), and each expert of the pass's union streams its
//             weights once for all rows that chose it.
// Both run the same 16-row MFMA tile code, so a row's output does not depend
// on which other rows share its tile: the two forms agree bitwise.  Outputs
// are combined per token in slot order (routed slots 0..top_k-1, then the
// shared experts) and added to the residual.
#include "device.h"

namespace ssd {

// Work unit: [0] expert (routed 0..E-1, shared E+s), [1] rows (1..16),
// [2..17] row codes m*slots + slot.  groups[0] = units, groups[1] = union
// size; units start at groups + 16.
constexpr int UNIT_INTS = 18;

// Router softmax and top-k of token m, on one wave (E <= 64 lanes): the
// softmax probabilities, then top_k rounds of a wave argmax (lowest index on
// ties); the gate is the probability at the chosen id, not renormalised.
// Injected ids keep the router's probabilities as gates.
__device__ __forceinline__ void route_token(const float* __restrict__ rlogits, int m, int E, int top_k,
                                            const int* __restrict__ inject, int* __restrict__ ids,
                                            float* __restrict__ gates, int* __restrict__ sid, int lane) {
  const float l = lane < E ? rlogits[(size_t)m * E + lane] : -INFINITY;
  float mx = l;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float p = lane < E ? expf(l - mx) : 0.f;
  float sum = p;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
  const float prob = p / sum;
  if (inject) {
    for (int j = 0; j < top_k; ++j) {
      const int e = inject[(size_t)m * top_k + j];
      const float g = __shfl(prob, e);
      if (lane == 0) {
        ids[(size_t)m * top_k + j] = e;
        gates[(size_t)m * top_k + j] = g;
        sid[m * top_k + j] = e;
      }
    }
    return;
  }
  float v = lane < E ? prob : -INFINITY;
  for (int j = 0; j < top_k; ++j) {
    float bv = v;
    int bi = lane;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) {
      ids[(size_t)m * top_k + j] = bi;
      gates[(size_t)m * top_k + j] = bv;
      sid[m * top_k + j] = bi;
    }
    if (lane == bi) v = -INFINITY;
  }
}

// Routing of the pass and its work units (see UNIT_INTS), one workgroup:
// each wave routes tokens wave, wave + 8, ... (route_token), keeping the
// expert ids (M * top_k <= 256 * 8) in LDS, so the counting and scatter loops
// read LDS; the units per expert are placed by a prefix sum over one wave
// (E <= 64).  Also the union size of the pass.
constexpr int GROUP_IDS_CAP = 2048;
__global__ __launch_bounds__(512) void moe_route_group_kernel(const float* __restrict__ rlogits, const int* __restrict__ inject,
                                                              int* __restrict__ ids, float* __restrict__ gates, int M,
                                                              int top_k, int E, int n_shared, int dedup,
                                                              int* __restrict__ groups, int* __restrict__ union_out,
                                                              const float* __restrict__ ss_in, int nss, int d,
                                                              float eps, float* __restrict__ rstd) {
  __shared__ int cnt[64], ubase[65];
  __shared__ int sid[GROUP_IDS_CAP];
  const int tid = threadIdx.x;
  const int slots = top_k + n_shared;
  const int P = M * top_k;   // <= GROUP_IDS_CAP (launch_moe checks)
  const int mchunks = (M + 15) / 16;
  int* units = groups + 16;
  for (int m = tid >> 6; m < M; m += 8) {
    route_token(rlogits, m, E, top_k, inject, ids, gates, sid, tid & 63);
    if (ss_in) {   // the token's 1/rms of the folded ffn norm, for the expert gate/up products
      const float f = norm_rstd(ss_in, nss, d, eps, true, m, tid & 63, norm_part(ss_in, nss, true, m, tid & 63));
      if ((tid & 63) == 0) rstd[m] = f;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 512) {
    int n = 0;
    for (int p = 0; p < P; ++p) n += sid[p] == e;
    cnt[e] = n;
  }
  __syncthreads();
  if (tid < 64) {
    const int c = tid < E ? cnt[tid] : 0;
    const int nu = dedup ? (c + 15) / 16 : 0;
    int incl = nu;   // inclusive prefix sum of the units over the experts
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    if (tid < E) ubase[tid] = incl - nu;
    const int U = __popcll(__ballot(c > 0));
    const int total = __shfl(incl, 63);
    if (tid == 0) {
      ubase[E] = total;
      const int routed = dedup ? total : P;
      groups[0] = routed + n_shared * mchunks;
      groups[1] = U;
      *union_out = U;
    }
  }
  __syncthreads();
  const int routed = dedup ? ubase[E] : P;
  if (dedup) {
    // pair p is the k-th pair (in pair order) choosing its expert e: it goes
    // to row k % 16 of unit ubase[e] + k / 16, whose header the first row writes
    for (int p = tid; p < P; p += blockDim.x) {
      const int e = sid[p];
      int k = 0;
      for (int q = 0; q < p; ++q) k += sid[q] == e;
      int* u = units + (size_t)(ubase[e] + k / 16) * UNIT_INTS;
      if (k % 16 == 0) {
        u[0] = e;
        u[1] = min(16, cnt[e] - k);
      }
      u[2 + k % 16] = (p / top_k) * slots + p % top_k;
    }
  } else {
    for (int p = tid; p < P; p += blockDim.x) {
      int* u = units + (size_t)p * UNIT_INTS;
      u[0] = sid[p];
      u[1] = 1;
      u[2] = (p / top_k) * slots + p % top_k;
    }
  }
  for (int i = tid; i < n_shared * mchunks; i += 512) {
    const int s = i / mchunks, ch = i % mchunks;
    int* u = units + (size_t)(routed + i) * UNIT_INTS;
    const int nr = min(16, M - ch * 16);
    u[0] = E + s;
    u[1] = nr;
    for (int r = 0; r < nr; ++r) u[2 + r] = (ch * 16 + r) * slots + top_k + s;
  }
}

// Expert GEMM over work units.  PHASE 0: act = silu(x.Wg^T) * (x.Wu^T) (bf16,
// row code's slot of the act buffer), both products times the row's 1/rms
// when the norm is folded (ss_in); PHASE 1: y = act . Wd^T (float32).
// A workgroup owns TPW output column tiles of 16 (grid: column tile groups x
// units; units past groups[0] exit); its 4 waves split K and each wave runs
// every tile of the group on its K range, reusing each A fragment for them.
// An element's arithmetic does not depend on TPW.
template <int PHASE, int TPW>
__global__ __launch_bounds__(256) void moe_gemm_kernel(MoeArgs a) {
  constexpr int NW = PHASE == 0 ? 2 : 1;
  constexpr int NS = NW * TPW;
  const int* groups = a.groups;
  const int unit = blockIdx.y;
  if (unit >= groups[0]) return;
  const int* u = groups + 16 + (size_t)unit * UNIT_INTS;
  const int eid = u[0], nr = u[1];
  const bool sh = eid >= a.E;
  const int e = sh ? eid - a.E : eid;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, kg = lane >> 4, t0 = blockIdx.x * TPW;
  const int slots = a.top_k + a.n_shared;
  const bool ok = c < nr;
  const int code = ok ? u[2 + c] : 0;
  // packed expert weights: per expert, gate/up interleaved [fe/16 tiles] or
  // down [d/16 tiles], tiles of 16 rows x 64 K-elements
  const uint16_t* xr;
  const uint16_t* wr[NS];
  int K;
  if (PHASE == 0) {
    K = a.d;
    xr = (const uint16_t*)a.X + (size_t)(code / slots) * a.d + kg * 16;
    const uint16_t* ex = (const uint16_t*)(sh ? a.sg : a.eg) + (size_t)e * 2 * a.fe * a.d;
#pragma unroll
    for (int j = 0; j < NS; ++j) wr[j] = ex + ((size_t)(t0 + j / NW) * (K >> 6) * 2 + j % NW) * PACK_TILE + 8 * lane;
  } else {
    K = a.fe;
    xr = (const uint16_t*)a.act + (size_t)code * a.fe + kg * 16;
    const uint16_t* ex = (const uint16_t*)(sh ? a.sd : a.ed) + (size_t)e * a.d * a.fe;
#pragma unroll
    for (int j = 0; j < NS; ++j) wr[j] = ex + (size_t)(t0 + j) * (K >> 6) * PACK_TILE + 8 * lane;
  }
  const int S = K >> 6;   // 64-element chunks
  const int s0 = (S * wave) >> 2, s1 = (S * (wave + 1)) >> 2;
  f32x4 acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // folded norm: this lane's row's 1/rms (per token, from the routing kernel),
  // loaded before the weight stream
  const bool fold = PHASE == 0 && a.ss_in != nullptr;
  const float rrow = fold && ok ? a.rstd[code / slots] : 1.0f;
  // a tile's chunks are NW tiles apart (gate/up interleaved), independent tiles
  // one tile apart.  Load batches of 4 chunks for gate/up, 2 for down: at 46
  // instead of 78 VGPRs the down workgroups are all resident at once
  // (measured on DeepSeek-V2-Lite shapes: the expert op at 8 rows 141.6 ->
  // 139.0 us per-slot, 86.6 -> 84.8 us dedup; shallower gate/up batches were
  // slower).  The batch depth never changes the accumulation order.
  mfma_stream<NS, true, PHASE == 0 ? 4 : 2, NW * PACK_TILE>(xr, ok, wr, s0, s1, acc);

  __shared__ f32x4 red[3][NS][64];
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < NS; ++j) red[wave - 1][j][lane] = acc[j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = ((acc[j] + red[0][j][lane]) + red[1][j][lane]) + red[2][j][lane];
  float rs[4];   // 1/rms of rows 4kg + i, from the lanes holding those rows
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] = __shfl(rrow, 4 * kg + i);
#pragma unroll
  for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kg + i;
      if (r >= nr) continue;
      const int rc = u[2 + r];
      const int n = (t0 + jt) * 16 + c;
      if (PHASE == 0) {
        const float g = fold ? acc[jt * NW][i] * rs[i] : acc[jt * NW][i];
        const float up = fold ? acc[jt * NW + NW - 1][i] * rs[i] : acc[jt * NW + NW - 1][i];
        ((uint16_t*)a.act)[(size_t)rc * a.fe + n] = f2bf(g / (1.0f + expf(-g)) * up);
      } else {
        a.slot_out[(size_t)rc * a.d + n] = acc[jt][i];
      }
    }
}

// x[m] += sum_j gate[m][j] * y[m][j] + sum_s y[m][top_k + s], in slot order.
// One thread per column, 16 runs of ssw columns per workgroup (grid: column
// groups x rows); every slot's load is issued before the arithmetic (slots
// <= 16).  With ss_out set it also leaves bf16(x * gain_next) and, per run of
// ssw columns, the sum of squares taken in column order.
constexpr int MOE_MAX_SLOTS = 16;
template <int SSW>
__global__ __launch_bounds__(16 * SSW) void moe_combine_kernel(MoeArgs a) {
  __shared__ float xs[16 * SSW];
  const int m = blockIdx.y, t = threadIdx.x;
  const int col = blockIdx.x * 16 * SSW + t;
  const bool ok = col < a.d;
  const int slots = a.top_k + a.n_shared;
  const float* y = a.slot_out + (size_t)m * slots * a.d + (ok ? col : 0);
  float ys[MOE_MAX_SLOTS], gs[8];
#pragma unroll
  for (int j = 0; j < MOE_MAX_SLOTS; ++j) ys[j] = j < slots ? y[(size_t)j * a.d] : 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) gs[j] = j < a.top_k ? a.gates[(size_t)m * a.top_k + j] : 0.f;
  const float r = ok ? a.resid[(size_t)m * a.d + col] : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < a.top_k) acc = fmaf(gs[j], ys[j], acc);
#pragma unroll
  for (int j = 0; j < MOE_MAX_SLOTS; ++j)
    if (j >= a.top_k && j < slots) acc += ys[j];
  const float xv = r + acc;
  if (ok) a.resid[(size_t)m * a.d + col] = xv;
  if (!a.ss_out) return;
  if (ok) ((uint16_t*)a.xg_out)[(size_t)m * a.d + col] = f2bf(xv * bf2f(((const uint16_t*)a.gain_next)[col]));
  xs[t] = xv;
  __syncthreads();
  if (t < 16) {
    const int c0 = blockIdx.x * 16 * SSW + t * SSW;
    if (c0 < a.d) {
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < SSW; ++i) q = fmaf(xs[t * SSW + i], xs[t * SSW + i], q);
      a.ss_out[(size_t)m * (a.d / SSW) + c0 / SSW] = q;
    }
  }
}

hipError_t launch_moe(int dtype, const MoeArgs& a, hipStream_t s) {
  if (dtype != 1) return hipErrorNotSupported;
  // the combine walks each row in runs of ssw columns (a residual tile width)
  if ((a.ssw != 16 && a.ssw != 10 && a.ssw != 8) || a.d % a.ssw != 0) return hipErrorInvalidValue;
  if (a.top_k > 8 || a.top_k + a.n_shared > MOE_MAX_SLOTS || a.M * a.top_k > GROUP_IDS_CAP) return hipErrorInvalidValue;
  GemmArgs r{};
  r.X = a.X; r.ldx = a.d; r.W0 = a.router; r.M = a.M; r.N = a.E; r.K = a.d; r.y = a.rlogits; r.ldy = a.E;
  r.ss_in = a.ss_in; r.nss = a.nss; r.eps = a.eps;   // folded norm: logits times the row's 1/rms
  hipError_t e = launch_gemm(1, EPI_F32, r, s);
  if (e != hipSuccess) return e;
  moe_route_group_kernel<<<1, 512, 0, s>>>(a.rlogits, a.inject, a.ids, a.gates, a.M, a.top_k, a.E, a.n_shared, a.dedup,
                                           a.groups, a.union_out, a.ss_in, a.nss, a.d, a.eps, a.rstd);
  const int max_units = a.M * a.top_k + ((a.M + 15) / 16) * a.n_shared;
  // one column tile per workgroup in both phases: 4 tiles per workgroup in the
  // down projection (one A read for them) measured slower (the dedup expert
  // op at 8 rows 86 -> 92 us): the fewer workgroups leave the stream short of
  // parallelism
  moe_gemm_kernel<0, 1><<<dim3(a.fe / 16, max_units), 256, 0, s>>>(a);
  moe_gemm_kernel<1, 1><<<dim3(a.d / 16, max_units), 256, 0, s>>>(a);
  const dim3 cg((a.d + 16 * a.ssw - 1) / (16 * a.ssw), a.M);
  if (a.ssw == 16) moe_combine_kernel<16><<<cg, 16 * 16, 0, s>>>(a);
  else if (a.ssw == 10) moe_combine_kernel<10><<<cg, 16 * 10, 0, s>>>(a);
  else moe_combine_kernel<8><<<cg, 16 * 8, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ssd
