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

// Router softmax and top-k, one wave per token (E <= 64 lanes).
__global__ __launch_bounds__(64) void moe_topk_kernel(const float* __restrict__ rlogits, int E, int top_k,
                                                      const int* __restrict__ inject, int* __restrict__ ids,
                                                      float* __restrict__ gates) {
  const int m = blockIdx.x, lane = threadIdx.x;
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
    }
    if (lane == bi) v = -INFINITY;
  }
}

// Work units of the pass (see UNIT_INTS) and the union size.
__global__ __launch_bounds__(256) void moe_group_kernel(const int* __restrict__ ids, int M, int top_k, int E,
                                                        int n_shared, int dedup, int* __restrict__ groups,
                                                        int* __restrict__ union_out) {
  __shared__ int cnt[64], ubase[65];
  const int tid = threadIdx.x;
  const int slots = top_k + n_shared;
  const int P = M * top_k;
  const int mchunks = (M + 15) / 16;
  int* units = groups + 16;
  for (int e = tid; e < E; e += 256) {
    int n = 0;
    for (int p = 0; p < P; ++p) n += ids[p] == e;
    cnt[e] = n;
  }
  __syncthreads();
  if (tid == 0) {
    int b = 0, U = 0;
    for (int e = 0; e < E; ++e) {
      ubase[e] = b;
      if (dedup) b += (cnt[e] + 15) / 16;
      U += cnt[e] > 0;
    }
    ubase[E] = b;
    const int routed = dedup ? b : P;
    groups[0] = routed + n_shared * mchunks;
    groups[1] = U;
    *union_out = U;
  }
  __syncthreads();
  const int routed = dedup ? ubase[E] : P;
  if (dedup) {
    for (int e = tid; e < E; e += 256) {
      if (!cnt[e]) continue;
      int k = 0;
      for (int p = 0; p < P; ++p) {
        if (ids[p] != e) continue;
        int* u = units + (size_t)(ubase[e] + k / 16) * UNIT_INTS;
        if (k % 16 == 0) {
          u[0] = e;
          u[1] = min(16, cnt[e] - k);
        }
        u[2 + k % 16] = (p / top_k) * slots + p % top_k;
        ++k;
      }
    }
  } else {
    for (int p = tid; p < P; p += 256) {
      int* u = units + (size_t)p * UNIT_INTS;
      u[0] = ids[p];
      u[1] = 1;
      u[2] = (p / top_k) * slots + p % top_k;
    }
  }
  for (int i = tid; i < n_shared * mchunks; i += 256) {
    const int s = i / mchunks, ch = i % mchunks;
    int* u = units + (size_t)(routed + i) * UNIT_INTS;
    const int nr = min(16, M - ch * 16);
    u[0] = E + s;
    u[1] = nr;
    for (int r = 0; r < nr; ++r) u[2 + r] = (ch * 16 + r) * slots + top_k + s;
  }
}

// Expert GEMM over work units.  PHASE 0: act = silu(x.Wg^T) * (x.Wu^T) (bf16,
// row code's slot of the act buffer); PHASE 1: y = act . Wd^T (float32).
// grid (output column tiles of 16, units); units past groups[0] exit.
template <int PHASE>
__global__ __launch_bounds__(256) void moe_gemm_kernel(MoeArgs a) {
  constexpr int NW = PHASE == 0 ? 2 : 1;
  const int* groups = a.groups;
  const int unit = blockIdx.y;
  if (unit >= groups[0]) return;
  const int* u = groups + 16 + (size_t)unit * UNIT_INTS;
  const int eid = u[0], nr = u[1];
  const bool sh = eid >= a.E;
  const int e = sh ? eid - a.E : eid;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, kg = lane >> 4, t = blockIdx.x;
  const int slots = a.top_k + a.n_shared;
  const bool ok = c < nr;
  const int code = ok ? u[2 + c] : 0;
  // packed expert weights: per expert, gate/up interleaved [fe/16 tiles] or
  // down [d/16 tiles], tiles of 16 rows x 64 K-elements
  const uint16_t* xr;
  const uint16_t* wr[NW];
  int K;
  if (PHASE == 0) {
    K = a.d;
    xr = (const uint16_t*)a.X + (size_t)(code / slots) * a.d + kg * 16;
    const uint16_t* ex = (const uint16_t*)(sh ? a.sg : a.eg) + (size_t)e * 2 * a.fe * a.d;
#pragma unroll
    for (int j = 0; j < NW; ++j) wr[j] = ex + ((size_t)t * (K >> 6) * 2 + j) * PACK_TILE + 8 * lane;
  } else {
    K = a.fe;
    xr = (const uint16_t*)a.act + (size_t)code * a.fe + kg * 16;
    const uint16_t* ex = (const uint16_t*)(sh ? a.sd : a.ed) + (size_t)e * a.d * a.fe;
    wr[0] = ex + (size_t)t * (K >> 6) * PACK_TILE + 8 * lane;
  }
  const int S = K >> 6;   // 64-element chunks
  const int s0 = (S * wave) >> 2, s1 = (S * (wave + 1)) >> 2;
  f32x4 acc[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  mfma_stream<NW, true, 4>(xr, ok, wr, s0, s1, acc);

  __shared__ f32x4 red[3][NW][64];
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < NW; ++j) red[wave - 1][j][lane] = acc[j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < NW; ++j) acc[j] = ((acc[j] + red[0][j][lane]) + red[1][j][lane]) + red[2][j][lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * kg + i;
    if (r >= nr) continue;
    const int rc = u[2 + r];
    const int n = t * 16 + c;
    if (PHASE == 0) {
      const float g = acc[0][i], up = acc[NW - 1][i];
      ((uint16_t*)a.act)[(size_t)rc * a.fe + n] = f2bf(g / (1.0f + expf(-g)) * up);
    } else {
      a.slot_out[(size_t)rc * a.d + n] = acc[0][i];
    }
  }
}

// x[m] += sum_j gate[m][j] * y[m][j] + sum_s y[m][top_k + s], in slot order.
// A thread owns ssw consecutive columns; with ss_out set it also leaves their
// sum of squares and bf16(x * gain_next) for the next layer's folded norm.
template <int SSW>
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs a) {
  const int m = blockIdx.x;
  const int slots = a.top_k + a.n_shared;
  const float* y = a.slot_out + (size_t)m * slots * a.d;
  for (int c0 = threadIdx.x * SSW; c0 < a.d; c0 += 256 * SSW) {
    float q = 0.f;
#pragma unroll
    for (int i = c0; i < c0 + SSW; ++i) {
      float acc = 0.f;
      for (int j = 0; j < a.top_k; ++j) acc += a.gates[(size_t)m * a.top_k + j] * y[(size_t)j * a.d + i];
      for (int s = 0; s < a.n_shared; ++s) acc += y[(size_t)(a.top_k + s) * a.d + i];
      const float xv = a.resid[(size_t)m * a.d + i] + acc;
      a.resid[(size_t)m * a.d + i] = xv;
      if (a.ss_out) {
        q = fmaf(xv, xv, q);
        ((uint16_t*)a.xg_out)[(size_t)m * a.d + i] = f2bf(xv * bf2f(((const uint16_t*)a.gain_next)[i]));
      }
    }
    if (a.ss_out) a.ss_out[(size_t)m * (a.d / SSW) + c0 / SSW] = q;
  }
}

hipError_t launch_moe(int dtype, const MoeArgs& a, hipStream_t s) {
  if (dtype != 1) return hipErrorNotSupported;
  // the combine walks each row in runs of ssw columns (a residual tile width)
  if ((a.ssw != 16 && a.ssw != 10 && a.ssw != 8) || a.d % a.ssw != 0) return hipErrorInvalidValue;
  GemmArgs r{};
  r.X = a.X; r.ldx = a.d; r.W0 = a.router; r.M = a.M; r.N = a.E; r.K = a.d; r.y = a.rlogits; r.ldy = a.E;
  hipError_t e = launch_gemm(1, EPI_F32, r, s);
  if (e != hipSuccess) return e;
  moe_topk_kernel<<<a.M, 64, 0, s>>>(a.rlogits, a.E, a.top_k, a.inject, a.ids, a.gates);
  moe_group_kernel<<<1, 256, 0, s>>>(a.ids, a.M, a.top_k, a.E, a.n_shared, a.dedup, a.groups, a.union_out);
  const int max_units = a.M * a.top_k + ((a.M + 15) / 16) * a.n_shared;
  moe_gemm_kernel<0><<<dim3(a.fe / 16, max_units), 256, 0, s>>>(a);
  moe_gemm_kernel<1><<<dim3(a.d / 16, max_units), 256, 0, s>>>(a);
  if (a.ssw == 16) moe_combine_kernel<16><<<a.M, 256, 0, s>>>(a);
  else if (a.ssw == 10) moe_combine_kernel<10><<<a.M, 256, 0, s>>>(a);
  else moe_combine_kernel<8><<<a.M, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ssd
