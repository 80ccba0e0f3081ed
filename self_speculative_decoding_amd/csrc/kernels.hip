// gfx950 (CDNA4) kernels of the greedy self-speculative decode step.
//
// Every reduction below has an order fixed by the shape and by the row's own
// position only, never by the number of rows in the pass.  A token decoded one
// row at a time and the same token verified inside a k+1 block therefore get
// bitwise-identical logits, which is what makes greedy self-speculation emit
// exactly the plain greedy sequence on the GPU (MLX layer-skip blog, "Code":
// the lossless check; mlx-dflash README: bit-for-bit parity with greedy).
#include "device.h"

namespace ssd {

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

template <int SSW>
__global__ __launch_bounds__(256) void embed_norm_kernel(const int* __restrict__ tok, const uint16_t* __restrict__ emb,
                                                         float* __restrict__ x, int d, const uint16_t* __restrict__ g,
                                                         uint16_t* __restrict__ xg, float* __restrict__ ss,
                                                         uint16_t* __restrict__ xgp) {
  const int m = blockIdx.x;
  const uint16_t* row = emb + (size_t)tok[m] * d;
  for (int c0 = threadIdx.x * SSW; c0 < d; c0 += 256 * SSW) {
    // every load before the first store and before the optional copy's
    // branch, so that they are all in flight together
    uint16_t e[SSW], gw[SSW], vg[SSW];
#pragma unroll
    for (int j = 0; j < SSW; ++j) {
      e[j] = row[c0 + j];
      gw[j] = g[c0 + j];
    }
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < SSW; ++j) {
      const float v = bf2f(e[j]);
      x[(size_t)m * d + c0 + j] = v;
      vg[j] = f2bf(v * bf2f(gw[j]));
      xg[(size_t)m * d + c0 + j] = vg[j];
      q = fmaf(v, v, q);
    }
    ss[(size_t)m * (d / SSW) + c0 / SSW] = q;
    if (xgp) {   // fragment-order copy (frag_index)
#pragma unroll
      for (int j = 0; j < SSW; ++j) xgp[frag_index(m, c0 + j, d)] = vg[j];
    }
  }
}

// ---------------------------------------------------------------------------
// RMSNorm: y = x / sqrt(mean(x^2) + eps) * g, stored in the activation type
// ---------------------------------------------------------------------------

template <typename E>
__global__ __launch_bounds__(1024) void rmsnorm_kernel(const float* __restrict__ x, int ldx,
                                                       const E* __restrict__ g, E* __restrict__ y,
                                                       int ldy, int d, float eps) {
  // lanes own 4 consecutive elements: i = 4*(t + 1024*j); d is a multiple of 4
  __shared__ float ws[16];
  const float* xr = x + (size_t)blockIdx.x * ldx;
  constexpr int J = 4;   // d <= 16384
  float4 v[J];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = 4 * (threadIdx.x + 1024 * j);
    v[j] = i < d ? *(const float4*)(xr + i) : float4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    s = fmaf(v[j].x, v[j].x, s);
    s = fmaf(v[j].y, v[j].y, s);
    s = fmaf(v[j].z, v[j].z, s);
    s = fmaf(v[j].w, v[j].w, s);
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  s = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) s += ws[w];
  const float r = 1.0f / sqrtf(s / (float)d + eps);
  E* yr = y + (size_t)blockIdx.x * ldy;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = 4 * (threadIdx.x + 1024 * j);
    if (i < d) {
      yr[i] = fromf<E>(v[j].x * r * tof(g[i]));
      yr[i + 1] = fromf<E>(v[j].y * r * tof(g[i + 1]));
      yr[i + 2] = fromf<E>(v[j].z * r * tof(g[i + 2]));
      yr[i + 3] = fromf<E>(v[j].w * r * tof(g[i + 3]));
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
// select.  Per-partition (max, sum, P.V) go to a partial buffer that
// attn_combine_kernel reduces in partition order.
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
    for (int e = tid * VEC; e < PT * HD; e += 256 * VEC) {
      const int key = e / HD;
      uint4 kv = {0u, 0u, 0u, 0u};
      if (key0 + key <= maxpos) kv = *(const uint4*)(kb + e);
      *(uint4*)(Ks + e) = kv;
    }
    // V cache rows are head dims ([dim][position]); Vs is [key][dim]
    const E* vb = (const E*)a.vc + (size_t)kvh * HD * a.max_ctx + key0;
    for (int e = tid; e < PT * HD; e += 256) {
      const int dim = e / PT, key = e % PT;
      Vs[key * HD + dim] = key0 + key <= maxpos ? vb[(size_t)dim * a.max_ctx + key] : fromf<E>(0.f);
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
    float* po = a.part_o + (((size_t)row * a.hq + head) * a.pstride + p) * HD + sub * SL;
#pragma unroll
    for (int d = 0; d < SL; ++d) po[d] = o[d];
    if (sub == 0) {
      float* pm = a.part_ml + (((size_t)row * a.hq + head) * a.pstride + p) * 2;
      pm[0] = mx;
      pm[1] = l;
    }
  }

}

// bf16 attention partition on MFMA 16x16x32, one wave per workgroup.
//
// grid (partition p, kv head, group of NT tiles of 16 query vectors
// qi = r*G + g: row r, query head g of the kv group).  Keys sit in the MFMA
// row dimension: S^T = K . Q^T takes K rows (key 16kt + c) and Q as operands
// straight from the caches, and lane (c, kg) then holds the scores of query c
// for keys 16kt + 4kg + i.  Those registers are already the B operand of
// O^T = V^T . P^T when K-step ks takes keys 32ks + 4kg + {0..3} and
// 32ks + 16 + 4kg + {0..3} in lane group kg; the V cache is stored transposed
// ([dim][position]) so that A gets the same keys as two 8-byte pieces.  O^T
// lands as lane (c, kg) holding dims 16dt + 4kg + i of query c.  No LDS, no
// barrier.  The row max and sum of a query are an in-lane pass in fixed order
// and a butterfly over its 4 lane groups.  P is split into bf16 hi + lo
// parts.  The wave loads the partition's K and V once for its NT query tiles
// (NT = 2 for passes of two or more tiles); every tile runs the same
// instruction sequence, so an output element does not depend on the number
// of rows in the pass or on the tile it shares a wave with.
// The value of lane ^ 16 and lane ^ 32 on the gfx950 permlane swaps (VALU,
// no LDS): the same partners, so the same results, as __shfl_xor(v, 16 / 32).
__device__ __forceinline__ float lane_xor16(float v, int lane) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 16) ? s[0] : s[1]);
}
__device__ __forceinline__ float lane_xor32(float v, int lane) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 32) ? s[0] : s[1]);
}

// XCD-aware grids (AttnArgs::xcd, kv heads a multiple of 8): workgroups go to
// the 8 XCDs in turn, so a 1-D launch whose workgroup L handles kv head
// L % 8 + 8 j keeps every partition of a kv head, and the combine of its
// query heads, on one XCD: the combine then reads the partials from that
// XCD's L2 (16-row verify on 8B shapes: attention + combine 11.5 -> 10.5 us,
// 4 rows 7.1 -> 6.8 us).  Splits L = x + 8 q into (kv head, the rest).
struct XcdSplit {
  int kvh, rest;
};
__device__ __forceinline__ XcdSplit attn_xcd_map(int L, int hkv) {
  const int x = L & 7, q = L >> 3, per = hkv >> 3;
  return XcdSplit{x + 8 * (q % per), q / per};
}

template <int G, int NT>
__global__ __launch_bounds__(64) void attn_mfma_kernel(AttnArgs a) {
  constexpr int HD = 128, PT = ATT_PT;
  int p = blockIdx.x, kvh = blockIdx.y, zt = blockIdx.z;
  if (a.xcd) {
    const XcdSplit xs = attn_xcd_map(blockIdx.x, a.hkv);
    kvh = xs.kvh;
    p = xs.rest % a.n_part;
    zt = xs.rest / a.n_part;
  }
  const int lane = threadIdx.x, c = lane & 15, kg = lane >> 4;
  const int st0 = a.state[0];   // position load issued first, used late
  const int key0 = p * PT;
  const size_t ldc = a.max_ctx;   // positions per cache row (multiple of PT)
  int qr[NT], qg[NT];
  bool qv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int qi = (zt * NT + t) * 16 + c;
    qv[t] = qi < a.M * G;
    qr[t] = qv[t] ? qi / G : 0;
    qg[t] = qv[t] ? qi % G : 0;
  }

  // every load up front: Q (B of S^T), K (A of S^T), V^T (A of O^T)
  uint4 qa[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint16_t* qp =
        (const uint16_t*)a.q + (size_t)qr[t] * a.hq * HD + (size_t)(kvh * G + qg[t]) * HD + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[t][ks] = *(const uint4*)(qp + 32 * ks);
  }
  const uint16_t* kb = (const uint16_t*)a.kc + ((size_t)kvh * ldc + key0 + c) * HD + 8 * kg;
  uint4 kf[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[kt][ks] = *(const uint4*)(kb + (size_t)16 * kt * HD + 32 * ks);
  // Q and K issue before V: the waits count loads in issue order, so S^T and
  // the softmax can run while V is still arriving
  __builtin_amdgcn_sched_barrier(0);
  const uint16_t* vb = (const uint16_t*)a.vc + ((size_t)kvh * HD + c) * ldc + key0 + 4 * kg;
  uint2 vf[8][2][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) vf[dt][ks][h] = *(const uint2*)(vb + (size_t)16 * dt * ldc + 32 * ks + 16 * h);
  // and all of them issue here, not next to their first use
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // The tiles' phases run side by side (both S^T, both softmaxes, both
  // O^T), so one tile's MFMA chains overlap the other's; each tile's own
  // instruction sequence is unchanged.
  int pos[NT];
  f32x4 sc[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    pos[t] = st0 + a.pos_off + qr[t];   // this lane's query position
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sc[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kt][ks]),
                                                            __builtin_bit_cast(bf16x8, qa[t][ks]), sc[t][kt], 0, 0, 0);
    }
  }
  // softmax over this partition's keys for query c
  float m[NT], l[NT];
  uint32_t ph[NT][2][4], pl[NT][2][4];   // P^T hi / lo fragments, bf16 pairs
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m[t] = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = qv[t] && key0 + 16 * kt + 4 * kg + i <= pos[t];
        m[t] = valid ? fmaxf(m[t], sc[t][kt][i] * a.scale_log2) : m[t];
      }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) m[t] = fmaxf(m[t], lane_xor16(m[t], lane));
#pragma unroll
  for (int t = 0; t < NT; ++t) m[t] = fmaxf(m[t], lane_xor32(m[t], lane));
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    l[t] = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        float pv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bool valid = qv[t] && key0 + 16 * kt + 4 * kg + i + u <= pos[t];
          pv[u] = valid ? exp2f(sc[t][kt][i + u] * a.scale_log2 - m[t]) : 0.f;
          l[t] += pv[u];
        }
        const uint16_t h0 = f2bf(pv[0]), h1 = f2bf(pv[1]);
        const uint16_t l0 = f2bf(pv[0] - bf2f(h0)), l1 = f2bf(pv[1] - bf2f(h1));
        // K-step kt/2; elements 0..3 from even kt, 4..7 from odd kt
        ph[t][kt >> 1][(kt & 1) * 2 + i / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        pl[t][kt >> 1][(kt & 1) * 2 + i / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) l[t] += lane_xor16(l[t], lane);
#pragma unroll
  for (int t = 0; t < NT; ++t) l[t] += lane_xor32(l[t], lane);

  // keys past the last row's position: P is 0 there; keep 0 * V finite
  // (selects only: entries at or below the position pass unchanged)
  {
    const int maxpos = st0 + a.pos_off + a.M - 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = key0 + 32 * ks + 16 * h + 4 * kg;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          uint2 v = vf[dt][ks][h];
          // zero the 16-bit entries past maxpos
          v.x = k > maxpos ? 0u : (k + 1 > maxpos ? (v.x & 0xffffu) : v.x);
          v.y = k + 2 > maxpos ? 0u : (k + 3 > maxpos ? (v.y & 0xffffu) : v.y);
          vf[dt][ks][h] = v;
        }
      }
  }
  f32x4 o[NT][8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint4 va = {vf[dt][ks][0].x, vf[dt][ks][0].y, vf[dt][ks][1].x, vf[dt][ks][1].y};
        const uint4 bh = {ph[t][ks][0], ph[t][ks][1], ph[t][ks][2], ph[t][ks][3]};
        const uint4 bl = {pl[t][ks][0], pl[t][ks][1], pl[t][ks][2], pl[t][ks][3]};
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                           __builtin_bit_cast(bf16x8, bh), o[t][dt], 0, 0, 0);
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                           __builtin_bit_cast(bf16x8, bl), o[t][dt], 0, 0, 0);
      }
    }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!qv[t] || key0 > pos[t]) continue;
    const int row = qr[t], head = kvh * G + qg[t];
    const size_t ph_i = ((size_t)row * a.hq + head) * a.pstride + p;
    float* po = a.part_o + ph_i * HD + 4 * kg;
    // the two-tile kernel (wide passes) streams its partials out with
    // nontemporal stores (16-row verify on 8B shapes: attention + combine
    // 17.0 -> 14.6 us); one-tile passes measured faster with plain stores
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if (NT == 2) __builtin_nontemporal_store(o[t][dt], (f32x4*)(po + 16 * dt));
      else *(f32x4*)(po + 16 * dt) = o[t][dt];
    }
    if (kg == 0) {
      a.part_ml[ph_i * 2] = m[t];
      a.part_ml[ph_i * 2 + 1] = l[t];
    }
  }
}

// Wave-wide sum and max on DPP lane moves (VALU, no LDS round trip):
// quad swaps, half-row and row mirrors, then the row 15 / row 31 broadcasts
// carry the partial results up to lane 63, which readlane returns to every
// lane.  Lanes a step does not write keep `old`: 0 for sums, the lane's own
// value for maxima.  A fixed order, the same for every call.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xb1, 0xf>(v, 0.f);    // quad_perm [1,0,3,2]
  v += dpp_move<0x4e, 0xf>(v, 0.f);    // quad_perm [2,3,0,1]
  v += dpp_move<0x141, 0xf>(v, 0.f);   // row_half_mirror
  v += dpp_move<0x140, 0xf>(v, 0.f);   // row_mirror
  v += dpp_move<0x142, 0xa>(v, 0.f);   // row_bcast15 into rows 1 and 3
  v += dpp_move<0x143, 0xc>(v, 0.f);   // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_move<0xb1, 0xf>(v, v));
  v = fmaxf(v, dpp_move<0x4e, 0xf>(v, v));
  v = fmaxf(v, dpp_move<0x141, 0xf>(v, v));
  v = fmaxf(v, dpp_move<0x140, 0xf>(v, v));
  v = fmaxf(v, dpp_move<0x142, 0xa>(v, v));
  v = fmaxf(v, dpp_move<0x143, 0xc>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Combine of the attention partitions: one workgroup per (row, head), one
// lane per head dim.  Row r at position pos uses partitions 0..pos/PT with
// weights w_p = exp2(m_p - max m): thread p holds partition p's (m, l), the
// max and sum(w_p l_p) are fixed DPP reductions over each wave, then the two
// waves' results added through LDS, and the
// outputs add w_p o_p in partition order.  The partial outputs are loaded (up
// to 48 at a time) together with the (m, l) pairs, before the position.
template <typename E>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  constexpr int B = 48;   // partials per load batch (3072 keys)
  __shared__ float sw[128];
  __shared__ float red[4];
  int row = blockIdx.x, head = blockIdx.y;
  if (a.xcd) {   // the attention's XCD-aware order (attn_xcd_map): query heads of one kv head together
    const int G = a.hq / a.hkv;
    const XcdSplit xs = attn_xcd_map(blockIdx.x, a.hkv);
    head = xs.kvh * G + xs.rest % G;
    row = xs.rest / G;
  }
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int st0 = a.state[0];   // position load issued first, used late
  const int npmax = a.n_part;   // partitions the attention launch covered (<= 128)
  const size_t stride = a.hd;   // partitions of one (row, head) are contiguous
  const float* po = a.part_o + ((size_t)row * a.hq + head) * a.pstride * a.hd + (t < a.hd ? t : 0);
  // loads issued unconditionally (indexes clamped to the launched partitions)
  float v[B];
#pragma unroll
  for (int j = 0; j < B; ++j) v[j] = po[(size_t)min(j, npmax - 1) * stride];
  const float* pm = a.part_ml + (((size_t)row * a.hq + head) * a.pstride + min(t, npmax - 1)) * 2;
  const float m_t = pm[0], l_t = pm[1];
  const int pos = st0 + a.pos_off + row;
  const int np = pos / ATT_PT + 1;
  const bool in = t < np;   // entries past the row's partitions are never used
  const float mx = wave_max_dpp(in ? m_t : -INFINITY);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  const float w = in ? exp2f(m_t - M) : 0.f;
  sw[t] = w;
  const float lw = wave_sum_dpp(in ? w * l_t : 0.f);
  if (lane == 0) red[2 + wave] = lw;
  __syncthreads();
  const float L = red[2] + red[3];
  if (t >= a.hd) return;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < B; ++j)
    if (j < np) acc += sw[j] * v[j];
  for (int p0 = B; p0 < np; p0 += B) {
#pragma unroll
    for (int j = 0; j < B; ++j) v[j] = p0 + j < np ? po[(size_t)(p0 + j) * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (p0 + j < np) acc += sw[p0 + j] * v[j];
  }
  const E ov = fromf<E>(acc / L);
  ((E*)a.out)[(size_t)row * a.hq * a.hd + (size_t)head * a.hd + t] = ov;
  if (sizeof(E) == 2 && a.out_p) ((E*)a.out_p)[frag_index(row, head * a.hd + t, a.hq * a.hd)] = ov;
}

// ---------------------------------------------------------------------------
// argmax per row (lowest index among equal maxima)
// ---------------------------------------------------------------------------

__device__ __forceinline__ void amax_merge(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

// plain row scan (float32 models)
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
  for (int o = 32; o > 0; o >>= 1) amax_merge(best, idx, __shfl_xor(best, o), __shfl_xor(idx, o));
  if ((threadIdx.x & 63) == 0) { bv[threadIdx.x >> 6] = best; bi[threadIdx.x >> 6] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w) amax_merge(best, idx, bv[w], bi[w]);
    out[blockIdx.x] = idx == 0x7fffffff ? 0 : idx;
  }
}

// reduce of the per-tile (max, index) pairs written by the LM head epilogue
__global__ __launch_bounds__(1024) void argmax_tiles_kernel(const float* __restrict__ pv, const int* __restrict__ pi,
                                                            int nt, int* __restrict__ out) {
  __shared__ float bv[16];
  __shared__ int bi[16];
  const float* rv = pv + (size_t)blockIdx.x * nt;
  const int* ri = pi + (size_t)blockIdx.x * nt;
  constexpr int J = 16;   // nt <= 16384
  float v[J];
  int id[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int t = threadIdx.x + 1024 * j;
    v[j] = t < nt ? rv[t] : -INFINITY;
    id[j] = t < nt ? ri[t] : 0x7fffffff;
  }
  float best = v[0];
  int idx = id[0];
#pragma unroll
  for (int j = 1; j < J; ++j) amax_merge(best, idx, v[j], id[j]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax_merge(best, idx, __shfl_xor(best, o), __shfl_xor(idx, o));
  if ((threadIdx.x & 63) == 0) { bv[threadIdx.x >> 6] = best; bi[threadIdx.x >> 6] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w) amax_merge(best, idx, bv[w], bi[w]);
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

// Streaming read of n16 16-byte words (achievable HBM read bandwidth): each
// lane keeps 8 loads in flight; one XOR per workgroup lands in sink.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                         unsigned* __restrict__ sink) {
  // the streaming pattern of the GEMMs: each wave reads its own contiguous
  // range, 1 KB per load instruction, nontemporal, 8 loads per batch
  const int lane = threadIdx.x & 63;
  const size_t waves = (size_t)gridDim.x * 4, gw = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t chunks = n16 / 64, per = (chunks + waves - 1) / waves;
  const size_t c0 = gw * per, c1 = c0 + per < chunks ? c0 + per : chunks;
  unsigned acc = 0;
  size_t c = c0;
  for (; c + 8 <= c1; c += 8) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ld16_nt((const uint16_t*)(src + (c + j) * 64 + lane));
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; c < c1; ++c) {
    const uint4 v = ld16_nt((const uint16_t*)(src + c * 64 + lane));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  acc = __reduce_xor_sync(0xffffffffffffffffull, acc);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void scale_bf16_kernel(const float* __restrict__ x, const uint16_t* __restrict__ g,
                                                         uint16_t* __restrict__ xg, int d, int n,
                                                         uint16_t* __restrict__ xgp) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const uint16_t v = f2bf(x[i] * bf2f(g[i % d]));
    xg[i] = v;
    if (xgp) xgp[frag_index(i / d, i % d, d)] = v;   // fragment-order copy (frag_index)
  }
}

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

hipError_t launch_embed_norm(const int* tok, const void* E, float* x, int d, int M, const void* gain, void* xg,
                             float* ss, int ssw, hipStream_t s, void* xgp) {
  if (d % ssw != 0) return hipErrorInvalidValue;
  const uint16_t *e16 = (const uint16_t*)E, *g16 = (const uint16_t*)gain;
  switch (ssw) {   // the residual tile widths (resid_tile_width)
    case 16: embed_norm_kernel<16><<<M, 256, 0, s>>>(tok, e16, x, d, g16, (uint16_t*)xg, ss, (uint16_t*)xgp); break;
    case 10: embed_norm_kernel<10><<<M, 256, 0, s>>>(tok, e16, x, d, g16, (uint16_t*)xg, ss, (uint16_t*)xgp); break;
    case 8: embed_norm_kernel<8><<<M, 256, 0, s>>>(tok, e16, x, d, g16, (uint16_t*)xg, ss, (uint16_t*)xgp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const float* x, int ldx, const void* g, void* y, int ldy, int d, float eps,
                          int M, hipStream_t s) {
  if (dtype) rmsnorm_kernel<uint16_t><<<M, 1024, 0, s>>>(x, ldx, (const uint16_t*)g, (uint16_t*)y, ldy, d, eps);
  else rmsnorm_kernel<float><<<M, 1024, 0, s>>>(x, ldx, (const float*)g, (float*)y, ldy, d, eps);
  return hipGetLastError();
}

#ifndef SSD_ATT_NT2_MIN   // 16-query tiles per KV head from which one wave takes two of them
#define SSD_ATT_NT2_MIN 2
#endif

template <typename E>
static hipError_t attn_dispatch(AttnArgs a, int n_part, int hd, hipStream_t s) {
  if (n_part < 1 || n_part > a.pstride) return hipErrorInvalidValue;
  a.n_part = n_part;
  a.xcd = 0;   // set below for the MFMA kernel's 1-D grids only
  const int G = a.hq / a.hkv;
  dim3 grid(n_part, a.hkv, (a.M + ROW_TILE - 1) / ROW_TILE);
  bool done = false;
  if (sizeof(E) == 2 && hd == 128) {
    // one wave per partition and 16 query vectors, or per 2 x 16 when the
    // pass has two or more such tiles (the partition's K and V loaded once)
    const int tiles = (a.M * G + 15) / 16;
    a.xcd = a.hkv % 8 == 0;
    const dim3 g1 = a.xcd ? dim3(n_part * a.hkv * tiles) : dim3(n_part, a.hkv, tiles);
    const dim3 g2 = a.xcd ? dim3(n_part * a.hkv * ((tiles + 1) / 2)) : dim3(n_part, a.hkv, (tiles + 1) / 2);
#define SSD_ATTM(Gv)                                                              \
    if (G == Gv) {                                                                \
      if (tiles >= SSD_ATT_NT2_MIN) attn_mfma_kernel<Gv, 2><<<g2, 64, 0, s>>>(a); \
      else attn_mfma_kernel<Gv, 1><<<g1, 64, 0, s>>>(a);                         \
      done = true;                                                                \
    }
    SSD_ATTM(1) SSD_ATTM(2) SSD_ATTM(4)
#undef SSD_ATTM
  }
#define SSD_ATT(HDv, Gv) \
  if (!done && hd == HDv && G == Gv) { attn_kernel<E, HDv, Gv><<<grid, 256, 0, s>>>(a); done = true; }
  SSD_ATT(64, 1) SSD_ATT(64, 2) SSD_ATT(64, 4) SSD_ATT(128, 1) SSD_ATT(128, 2) SSD_ATT(128, 4)
#undef SSD_ATT
  if (!done) return hipErrorInvalidValue;
  attn_combine_kernel<E><<<a.xcd ? dim3(a.M * a.hq) : dim3(a.M, a.hq), 128, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnArgs& a, int n_part, hipStream_t s) {
  return dtype ? attn_dispatch<uint16_t>(a, n_part, a.hd, s) : attn_dispatch<float>(a, n_part, a.hd, s);
}

hipError_t launch_argmax(const float* logits, int V, int ld, int* out, int M, hipStream_t s) {
  argmax_kernel<<<M, 1024, 0, s>>>(logits, V, ld, out);
  return hipGetLastError();
}

hipError_t launch_argmax_tiles(const float* pv, const int* pi, int nt, int* out, int M, hipStream_t s) {
  argmax_tiles_kernel<<<M, 1024, 0, s>>>(pv, pi, nt, out);
  return hipGetLastError();
}

hipError_t launch_accept(int* block, const int* post, int k, int* state, int* outlog, int* result,
                         hipStream_t s) {
  accept_kernel<<<1, 64, 0, s>>>(block, post, k, state, outlog, result);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, size_t bytes, unsigned* sink, int blocks, hipStream_t s) {
  read_probe_kernel<<<blocks, 256, 0, s>>>((const uint4*)src, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_set_state(int* state, int idx, int value, hipStream_t s) {
  set_state_kernel<<<1, 1, 0, s>>>(state, idx, value);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t s) {
  copy_f32_kernel<<<(n + 255) / 256, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

hipError_t launch_scale_bf16(const float* x, const void* g, void* xg, int d, int M, hipStream_t s, void* xgp) {
  const int n = d * M;
  scale_bf16_kernel<<<(n + 255) / 256, 256, 0, s>>>(x, (const uint16_t*)g, (uint16_t*)xg, d, n, (uint16_t*)xgp);
  return hipGetLastError();
}

hipError_t launch_copy_tokens(const int* src, int* dst, int n, hipStream_t s) {
  copy_tokens_kernel<<<1, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}


}  // namespace ssd
