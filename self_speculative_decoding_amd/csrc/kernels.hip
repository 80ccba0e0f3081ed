// gfx950 (CDNA4) kernels of the greedy self-speculative decode step.
//
// Every reduction below has an order fixed by the shape and by the row's own
// position only, never by the number of rows in the pass.  A token decoded one
// row at a time and the same token verified inside a k+1 block therefore get
// bitwise-identical logits, which is what makes greedy self-speculation emit
// exactly the plain greedy sequence on the GPU (MLX layer-skip blog, "Code":
// the lossless check; mlx-dflash README: bit-for-bit parity with greedy).
#include "kernels.h"

#include <math.h>

namespace ssd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// ---------------------------------------------------------------------------
// element helpers (bf16 is carried as uint16 bit patterns)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {   // nearest, ties to even
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float tof(float v) { return v; }
__device__ __forceinline__ float tof(uint16_t v) { return bf2f(v); }
template <typename E> __device__ __forceinline__ E fromf(float v);
template <> __device__ __forceinline__ float fromf<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t fromf<uint16_t>(float v) { return f2bf(v); }

__device__ __forceinline__ float wave_sum(float v) {   // fixed butterfly, same result in all lanes
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// embedding gather: x[m, :] = E[tok[m], :] as float32 (residual stream)
// ---------------------------------------------------------------------------

template <typename E>
__global__ __launch_bounds__(256) void embed_kernel(const int* __restrict__ tok, const E* __restrict__ emb,
                                                    float* __restrict__ x, int d) {
  const int m = blockIdx.x;
  const E* row = emb + (size_t)tok[m] * d;
  for (int i = threadIdx.x; i < d; i += 256) x[(size_t)m * d + i] = tof(row[i]);
}

// ---------------------------------------------------------------------------
// RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, stored in the activation type
// ---------------------------------------------------------------------------

template <typename E>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int ldx,
                                                      const E* __restrict__ g, E* __restrict__ y,
                                                      int ldy, int d, float eps) {
  __shared__ float ws[4];
  const float* xr = x + (size_t)blockIdx.x * ldx;
  float s = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) s = fmaf(xr[i], xr[i], s);
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  s = ((ws[0] + ws[1]) + ws[2]) + ws[3];
  const float r = 1.0f / sqrtf(s / (float)d + eps);
  E* yr = y + (size_t)blockIdx.x * ldy;
  for (int i = threadIdx.x; i < d; i += 256) yr[i] = fromf<E>(xr[i] * r * tof(g[i]));
}

// ---------------------------------------------------------------------------
// GEMM epilogues
// ---------------------------------------------------------------------------

template <typename E>
__device__ __forceinline__ void epi_single(const GemmArgs& a, int epi, int m, int n, float v) {
  if (epi == EPI_F32) {
    a.y[(size_t)m * a.ldy + n] = v;
  } else if (epi == EPI_RESID) {
    const float r = a.y[(size_t)m * a.ldy + n] + v;
    a.y[(size_t)m * a.ldy + n] = r;
    if (a.tap) ((E*)a.tap)[(size_t)m * a.ldtap + n] = fromf<E>(r);
  } else {  // EPI_STORE
    ((E*)a.out)[(size_t)m * a.ldo + n] = fromf<E>(v);
  }
}

template <typename E>
__device__ __forceinline__ void epi_swiglu(const GemmArgs& a, int m, int n, float g, float u) {
  const float s = g / (1.0f + expf(-g));
  ((E*)a.out)[(size_t)m * a.ldo + n] = fromf<E>(s * u);
}

// (v0, v1) are dims (i, i + hd/2) of output head `head` of [q | k | v]
template <typename E>
__device__ __forceinline__ void epi_qkv_pair(const GemmArgs& a, int m, int head, int i, float v0, float v1) {
  const int half = a.hd >> 1;
  const int pos = a.state[0] + a.pos_off + m;
  if (head < a.hq + a.hkv) {
    const float c = a.cos_t[(size_t)pos * half + i], s = a.sin_t[(size_t)pos * half + i];
    const float o0 = v0 * c - v1 * s, o1 = v1 * c + v0 * s;
    E* dst = head < a.hq ? (E*)a.q + (size_t)m * a.hq * a.hd + (size_t)head * a.hd
                         : (E*)a.kc + ((size_t)(head - a.hq) * a.max_ctx + pos) * a.hd;
    dst[i] = fromf<E>(o0);
    dst[i + half] = fromf<E>(o1);
  } else {
    E* dst = (E*)a.vc + ((size_t)(head - a.hq - a.hkv) * a.max_ctx + pos) * a.hd;
    dst[i] = fromf<E>(v0);
    dst[i + half] = fromf<E>(v1);
  }
}

template <typename E>
__device__ __forceinline__ void epi_v_single(const GemmArgs& a, int m, int vh, int dim, float v) {
  const int pos = a.state[0] + a.pos_off + m;
  ((E*)a.vc)[((size_t)vh * a.max_ctx + pos) * a.hd + dim] = fromf<E>(v);
}

// ---------------------------------------------------------------------------
// bf16 skinny GEMM on MFMA 16x16x32 (weight streaming)
//
// Y[M,N] = X[M,K] . W[N,K]^T, M padded to 16-row tiles (grid.y).  A workgroup
// of 4 waves owns NW 16-column tiles; the waves split K into 4 contiguous
// quarters, each accumulating its MFMA K-steps in order, and the quarters are
// added in wave order through LDS.  The per-element arithmetic is therefore a
// function of (shape, row data) only.  Each lane streams 16-byte pieces of
// weight rows; U K-steps of loads are issued before their MFMAs.
//
// MFMA 16x16x32 bf16 lane layout: A row = lane%16, B column = lane%16, both
// with the same 8-element K group lane/16; D: column lane%16, rows
// 4*(lane/16) .. +3.
// ---------------------------------------------------------------------------

constexpr int GEMM_U = 8;

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *(const uint4*)p; }

template <int EPI, int NW>
__device__ __forceinline__ const uint16_t* gemm_row(const GemmArgs& a, int t, int j, int c, int* head_out,
                                                    int* dim_out) {
  if (EPI == EPI_QKV) {
    const int col0 = t * 16;
    const int head = col0 / a.hd, jj = (col0 % a.hd) / 16, half = a.hd >> 1;
    int dim;
    if (head < a.hq + a.hkv) dim = c < 8 ? 8 * jj + c : half + 8 * jj + (c - 8);
    else dim = 16 * jj + c;
    *head_out = head;
    *dim_out = dim;
    if (head < a.hq) return (const uint16_t*)a.W0 + ((size_t)head * a.hd + dim) * a.K;
    if (head < a.hq + a.hkv) return (const uint16_t*)a.W1 + ((size_t)(head - a.hq) * a.hd + dim) * a.K;
    return (const uint16_t*)a.W2 + ((size_t)(head - a.hq - a.hkv) * a.hd + dim) * a.K;
  }
  const uint16_t* W = (const uint16_t*)(j == 0 ? a.W0 : a.W1);
  return W + (size_t)(t * 16 + c) * a.K;
}

template <int EPI, int NW>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, kg = lane >> 4;
  const int t = blockIdx.x, mt = blockIdx.y;
  const int am = mt * 16 + c;
  const bool av_ok = am < a.M;
  const uint16_t* xr = (const uint16_t*)a.X + (size_t)(av_ok ? am : 0) * a.ldx + kg * 8;
  const uint16_t* wr[NW];
  int head = 0, dim = 0;
#pragma unroll
  for (int j = 0; j < NW; ++j) wr[j] = gemm_row<EPI, NW>(a, t, j, c, &head, &dim) + kg * 8;

  const int S = a.K >> 5;
  const int s0 = (S * wave) >> 2, s1 = (S * (wave + 1)) >> 2;
  f32x4 acc[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint4 zero = {0u, 0u, 0u, 0u};

  int s = s0;
  for (; s + GEMM_U <= s1; s += GEMM_U) {
    uint4 xa[GEMM_U], wb[NW][GEMM_U];
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
#pragma unroll
      for (int j = 0; j < NW; ++j) wb[j][u] = ld16(wr[j] + (size_t)(s + u) * 32);
      xa[u] = av_ok ? ld16(xr + (size_t)(s + u) * 32) : zero;
    }
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u)
#pragma unroll
      for (int j = 0; j < NW; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[u]),
                                                         __builtin_bit_cast(bf16x8, wb[j][u]), acc[j], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    uint4 xa = av_ok ? ld16(xr + (size_t)s * 32) : zero;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      uint4 wb = ld16(wr[j] + (size_t)s * 32);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                       __builtin_bit_cast(bf16x8, wb), acc[j], 0, 0, 0);
    }
  }

  __shared__ f32x4 red[3][NW][64];
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < NW; ++j) red[wave - 1][j][lane] = acc[j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < NW; ++j) acc[j] = ((acc[j] + red[0][j][lane]) + red[1][j][lane]) + red[2][j][lane];

  if (EPI == EPI_QKV) {
    const bool rot = head < a.hq + a.hkv;
    float part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) part[i] = __shfl_xor(acc[0][i], 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * kg + i;
      if (m >= a.M) continue;
      if (rot) {
        if (c < 8) epi_qkv_pair<uint16_t>(a, m, head, dim, acc[0][i], part[i]);
      } else {
        epi_v_single<uint16_t>(a, m, head - a.hq - a.hkv, dim, acc[0][i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * kg + i;
      if (m >= a.M) continue;
      const int n = t * 16 + c;
      if (EPI == EPI_SWIGLU) epi_swiglu<uint16_t>(a, m, n, acc[0][i], acc[1][i]);
      else epi_single<uint16_t>(a, EPI, m, n, acc[0][i]);
    }
  }
}

// ---------------------------------------------------------------------------
// float32 GEMM on the vector ALU (small float32 models)
//
// One wave owns one output pair: (i, i + hd/2) of a q/k/v head for QKV,
// (gate i, up i) for SwiGLU, (2i, 2i+1) otherwise.  Lanes stride over K in
// order and a fixed butterfly adds the lane partials.
// ---------------------------------------------------------------------------

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pi = blockIdx.x * 4 + wave;
  int npairs, head = 0, i = 0;
  const float *w0, *w1;
  if (EPI == EPI_QKV) {
    const int half = a.hd >> 1;
    npairs = (a.hq + 2 * a.hkv) * half;
    if (pi >= npairs) return;
    head = pi / half;
    i = pi % half;
    const float* W;
    size_t r;
    if (head < a.hq) { W = (const float*)a.W0; r = (size_t)head * a.hd + i; }
    else if (head < a.hq + a.hkv) { W = (const float*)a.W1; r = (size_t)(head - a.hq) * a.hd + i; }
    else { W = (const float*)a.W2; r = (size_t)(head - a.hq - a.hkv) * a.hd + i; }
    w0 = W + r * a.K;
    w1 = W + (r + half) * a.K;
  } else if (EPI == EPI_SWIGLU) {
    npairs = a.N;
    if (pi >= npairs) return;
    w0 = (const float*)a.W0 + (size_t)pi * a.K;
    w1 = (const float*)a.W1 + (size_t)pi * a.K;
  } else {
    npairs = a.N >> 1;
    if (pi >= npairs) return;
    w0 = (const float*)a.W0 + (size_t)(2 * pi) * a.K;
    w1 = w0 + a.K;
  }
  const int m1 = min(a.M, (int)(blockIdx.y + 1) * 16);
  for (int m = blockIdx.y * 16; m < m1; ++m) {
    const float* xr = (const float*)a.X + (size_t)m * a.ldx;
    float s0 = 0.f, s1 = 0.f;
    for (int k = lane; k < a.K; k += 64) {
      const float xv = xr[k];
      s0 = fmaf(xv, w0[k], s0);
      s1 = fmaf(xv, w1[k], s1);
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if (lane == 0) {
      if (EPI == EPI_QKV) epi_qkv_pair<float>(a, m, head, i, s0, s1);
      else if (EPI == EPI_SWIGLU) epi_swiglu<float>(a, m, pi, s0, s1);
      else {
        epi_single<float>(a, EPI, m, 2 * pi, s0);
        epi_single<float>(a, EPI, m, 2 * pi + 1, s1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode attention over the KV cache, causal inside the block
//
// grid (partition p, kv head, 16-row tile).  A workgroup stages the K and V
// rows of its partition [p*PT, p*PT+PT) in LDS and serves the 16 rows x G query
// heads of its tile (G = hq/hkv).  TPQ = 256/(16 G) lanes share one query
// vector, each holding a fixed slice of head dims: a dot product is the
// in-order slice sum followed by a fixed butterfly over the TPQ lanes, so all
// lanes hold all PT scores.  Keys past the row's own position are excluded by
// select.  Per-partition (max, sum, P.V) go to a partial buffer; the last
// workgroup of a (kv head, tile) to finish (atomic ticket) combines the
// partitions 0..pos/PT of each row in partition order.
// ---------------------------------------------------------------------------

template <typename E, int HD, int G>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int PT = ATT_PT;
  constexpr int QV = ROW_TILE * G;        // query vectors per workgroup
  constexpr int TPQ = 256 / QV;           // lanes per query vector (same wave)
  constexpr int SL = HD / TPQ;            // head dims per lane
  constexpr int VEC = 16 / sizeof(E);     // elements per 16-byte load
  __shared__ __attribute__((aligned(16))) E Ks[PT * HD];
  __shared__ __attribute__((aligned(16))) E Vs[PT * HD];
  __shared__ float S[QV][PT + 1];
  __shared__ int ticket;

  const int p = blockIdx.x, kvh = blockIdx.y, mt = blockIdx.z;
  const int tid = threadIdx.x;
  const int base = a.state[0] + a.pos_off;
  const int row0 = mt * ROW_TILE;
  const int nrows = min(ROW_TILE, a.M - row0);
  const int key0 = p * PT;
  const int maxpos = base + row0 + nrows - 1;
  const bool active = key0 <= maxpos;

  if (active) {
    const E* kb = (const E*)a.kc + ((size_t)kvh * a.max_ctx + key0) * HD;
    const E* vb = (const E*)a.vc + ((size_t)kvh * a.max_ctx + key0) * HD;
    for (int e = tid * VEC; e < PT * HD; e += 256 * VEC) {
      const int key = e / HD;
      uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key0 + key <= maxpos) {
        kv = *(const uint4*)(kb + e);
        vv = *(const uint4*)(vb + e);
      }
      *(uint4*)(Ks + e) = kv;
      *(uint4*)(Vs + e) = vv;
    }
  }
  __syncthreads();

  const int qi = tid / TPQ, sub = tid % TPQ;
  const int r = qi / G, g = qi % G;
  const int head = kvh * G + g;
  const int row = row0 + r;
  const int pos = base + row;
  const bool qok = active && r < nrows && key0 <= pos;

  float mx = -INFINITY, l = 0.f;
  if (qok) {
    float q[SL];
    const E* qp = (const E*)a.q + (size_t)row * a.hq * HD + (size_t)head * HD + sub * SL;
#pragma unroll
    for (int d = 0; d < SL; ++d) q[d] = tof(qp[d]);
#pragma unroll 2
    for (int kk = 0; kk < PT; ++kk) {
      const E* kr = Ks + kk * HD + sub * SL;
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < SL; ++d) acc = fmaf(q[d], tof(kr[d]), acc);
#pragma unroll
      for (int o = 1; o < TPQ; o <<= 1) acc += __shfl_xor(acc, o);
      const bool valid = key0 + kk <= pos;
      const float sv = acc * a.scale_log2;
      mx = valid ? fmaxf(mx, sv) : mx;
      if ((kk % TPQ) == sub) S[qi][kk] = sv;
    }
  }
  __syncthreads();
  if (qok) {
    // probabilities of this lane's keys kk = sub + j*TPQ, partial sums in j order
#pragma unroll 4
    for (int j = 0; j < PT / TPQ; ++j) {
      const int kk = sub + j * TPQ;
      const bool valid = key0 + kk <= pos;
      const float pv = valid ? exp2f(S[qi][kk] - mx) : 0.f;
      S[qi][kk] = pv;
      l += pv;
    }
#pragma unroll
    for (int o = 1; o < TPQ; o <<= 1) l += __shfl_xor(l, o);
  }
  __syncthreads();
  if (qok) {
    float o[SL];
#pragma unroll
    for (int d = 0; d < SL; ++d) o[d] = 0.f;
#pragma unroll 2
    for (int kk = 0; kk < PT; ++kk) {
      const bool valid = key0 + kk <= pos;
      const float pv = S[qi][kk];
      const E* vr = Vs + kk * HD + sub * SL;
#pragma unroll
      for (int d = 0; d < SL; ++d) o[d] += valid ? pv * tof(vr[d]) : 0.f;
    }
    float* po = a.part_o + (((size_t)p * a.R + row) * a.hq + head) * HD + sub * SL;
#pragma unroll
    for (int d = 0; d < SL; ++d) po[d] = o[d];
    if (sub == 0) {
      float* pm = a.part_ml + (((size_t)p * a.R + row) * a.hq + head) * 2;
      pm[0] = mx;
      pm[1] = l;
    }
  }

  // the last workgroup of this (kv head, row tile) to finish combines the partitions
  __threadfence();
  __syncthreads();
  if (tid == 0) ticket = atomicAdd(a.counters + kvh * (a.R / ROW_TILE) + mt, 1);
  __syncthreads();
  if (ticket != (int)gridDim.x - 1) return;
  __threadfence();
  if (tid == 0) a.counters[kvh * (a.R / ROW_TILE) + mt] = 0;

  if (r < nrows) {
    const int np = pos / PT + 1;
    float M = -INFINITY;
    for (int pp = 0; pp < np; ++pp)
      M = fmaxf(M, a.part_ml[(((size_t)pp * a.R + row) * a.hq + head) * 2]);
    float L = 0.f, o[SL];
#pragma unroll
    for (int d = 0; d < SL; ++d) o[d] = 0.f;
    for (int pp = 0; pp < np; ++pp) {
      const float* pm = a.part_ml + (((size_t)pp * a.R + row) * a.hq + head) * 2;
      const float w = exp2f(pm[0] - M);
      L += w * pm[1];
      const float* po = a.part_o + (((size_t)pp * a.R + row) * a.hq + head) * HD + sub * SL;
#pragma unroll
      for (int d = 0; d < SL; ++d) o[d] += w * po[d];
    }
    const float inv = 1.0f / L;
    E* out = (E*)a.out + (size_t)row * a.hq * HD + (size_t)head * HD + sub * SL;
#pragma unroll
    for (int d = 0; d < SL; ++d) out[d] = fromf<E>(o[d] * inv);
  }
}

// ---------------------------------------------------------------------------
// argmax per row (lowest index among equal maxima)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ L, int V, int ld,
                                                      int* __restrict__ out) {
  __shared__ float bv[16];
  __shared__ int bi[16];
  const float* row = L + (size_t)blockIdx.x * ld;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int v = threadIdx.x; v < V; v += 1024) {
    const float x = row[v];
    if (x > best) { best = x; idx = v; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(idx, o);
    if (ob > best || (ob == best && oi < idx)) { best = ob; idx = oi; }
  }
  if ((threadIdx.x & 63) == 0) { bv[threadIdx.x >> 6] = best; bi[threadIdx.x >> 6] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w)
      if (bv[w] > best || (bv[w] == best && bi[w] < idx)) { best = bv[w]; idx = bi[w]; }
    out[blockIdx.x] = idx == 0x7fffffff ? 0 : idx;
  }
}

// ---------------------------------------------------------------------------
// greedy accept + rollback, one wave
//
// block = [t_last, d_1..d_k], post = [p_0..p_k].  a = number of leading i with
// d_{i+1} == p_i (the cumulative product of the match bits, read off the
// wave's ballot of mismatches).  Emits d_1..d_a, p_a; the committed length
// (state[0]) advances by a+1; p_a becomes the new t_last.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(64) void accept_kernel(int* block, const int* post, int k, int* state,
                                                    int* outlog, int* result) {
  const int l = threadIdx.x;
  const bool mism = l < k && block[1 + l] != post[l];
  const unsigned long long b = __ballot(mism) | (1ull << k);
  const int a = __builtin_ctzll(b);
  const int base = state[1];
  if (l <= a) {
    const int tok = l < a ? block[1 + l] : post[a];
    result[2 + l] = tok;
    outlog[base + l] = tok;
  }
  if (l == 0) {
    result[0] = a;
    result[1] = a + 1;
    state[0] += a + 1;
    state[1] += a + 1;
    block[0] = post[a];
  }
}

__global__ void set_state_kernel(int* state, int idx, int value) { state[idx] = value; }

__global__ void copy_tokens_kernel(const int* src, int* dst, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_embed(int dtype, const int* tok, const void* E, float* x, int d, int M, hipStream_t s) {
  if (dtype) embed_kernel<uint16_t><<<M, 256, 0, s>>>(tok, (const uint16_t*)E, x, d);
  else embed_kernel<float><<<M, 256, 0, s>>>(tok, (const float*)E, x, d);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const float* x, int ldx, const void* g, void* y, int ldy, int d, float eps,
                          int M, hipStream_t s) {
  if (dtype) rmsnorm_kernel<uint16_t><<<M, 256, 0, s>>>(x, ldx, (const uint16_t*)g, (uint16_t*)y, ldy, d, eps);
  else rmsnorm_kernel<float><<<M, 256, 0, s>>>(x, ldx, (const float*)g, (float*)y, ldy, d, eps);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s) {
  const int mt = (a.M + 15) / 16;
  if (dtype) {
    int tiles;
    if (epi == EPI_QKV) tiles = (a.hq + 2 * a.hkv) * a.hd / 16;
    else tiles = a.N / 16;
    dim3 grid(tiles, mt);
    switch (epi) {
      case EPI_F32: gemm_bf16_kernel<EPI_F32, 1><<<grid, 256, 0, s>>>(a); break;
      case EPI_RESID: gemm_bf16_kernel<EPI_RESID, 1><<<grid, 256, 0, s>>>(a); break;
      case EPI_SWIGLU: gemm_bf16_kernel<EPI_SWIGLU, 2><<<grid, 256, 0, s>>>(a); break;
      case EPI_QKV: gemm_bf16_kernel<EPI_QKV, 1><<<grid, 256, 0, s>>>(a); break;
      case EPI_STORE: gemm_bf16_kernel<EPI_STORE, 1><<<grid, 256, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    int npairs;
    if (epi == EPI_QKV) npairs = (a.hq + 2 * a.hkv) * (a.hd / 2);
    else if (epi == EPI_SWIGLU) npairs = a.N;
    else npairs = a.N / 2;
    dim3 grid((npairs + 3) / 4, mt);
    switch (epi) {
      case EPI_F32: gemm_f32_kernel<EPI_F32><<<grid, 256, 0, s>>>(a); break;
      case EPI_RESID: gemm_f32_kernel<EPI_RESID><<<grid, 256, 0, s>>>(a); break;
      case EPI_SWIGLU: gemm_f32_kernel<EPI_SWIGLU><<<grid, 256, 0, s>>>(a); break;
      case EPI_QKV: gemm_f32_kernel<EPI_QKV><<<grid, 256, 0, s>>>(a); break;
      case EPI_STORE: gemm_f32_kernel<EPI_STORE><<<grid, 256, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <typename E>
static hipError_t attn_dispatch(const AttnArgs& a, int n_part, int hd, hipStream_t s) {
  const int G = a.hq / a.hkv;
  dim3 grid(n_part, a.hkv, (a.M + ROW_TILE - 1) / ROW_TILE);
#define SSD_ATT(HDv, Gv) \
  if (hd == HDv && G == Gv) { attn_kernel<E, HDv, Gv><<<grid, 256, 0, s>>>(a); return hipGetLastError(); }
  SSD_ATT(64, 1) SSD_ATT(64, 2) SSD_ATT(64, 4) SSD_ATT(128, 1) SSD_ATT(128, 2) SSD_ATT(128, 4)
#undef SSD_ATT
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int dtype, const AttnArgs& a, int n_part, hipStream_t s) {
  return dtype ? attn_dispatch<uint16_t>(a, n_part, a.hd, s) : attn_dispatch<float>(a, n_part, a.hd, s);
}

hipError_t launch_argmax(const float* logits, int V, int ld, int* out, int M, hipStream_t s) {
  argmax_kernel<<<M, 1024, 0, s>>>(logits, V, ld, out);
  return hipGetLastError();
}

hipError_t launch_accept(int* block, const int* post, int k, int* state, int* outlog, int* result,
                         hipStream_t s) {
  accept_kernel<<<1, 64, 0, s>>>(block, post, k, state, outlog, result);
  return hipGetLastError();
}

hipError_t launch_set_state(int* state, int idx, int value, hipStream_t s) {
  set_state_kernel<<<1, 1, 0, s>>>(state, idx, value);
  return hipGetLastError();
}

hipError_t launch_copy_tokens(const int* src, int* dst, int n, hipStream_t s) {
  copy_tokens_kernel<<<1, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

hipError_t launch_moe(int, const MoeArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ssd
