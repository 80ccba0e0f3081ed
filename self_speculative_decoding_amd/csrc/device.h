// Device-side helpers shared by the gfx950 kernel files.
#pragma once
#include <math.h>

#include "kernels.h"

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


__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *(const uint4*)p; }

// Weights are read once per pass: nontemporal loads stream them without
// allocating in the caches.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const uint16_t* p) {
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return uint4{t[0], t[1], t[2], t[3]};
}

// Folded RMSNorm (GemmArgs::ss_in): the 1/rms factor of row m of K columns
// from its nss sums-of-squares partials (one per residual tile).  Lane l
// holds partials 4l..4l+3; partials from 256 on are added after, 64 apart;
// then a fixed butterfly over the wave: the order is fixed by nss alone,
// whatever the pass width.  Every lane of the wave calls both; rows with
// ok == false read nothing.
__device__ __forceinline__ float4 norm_part(const float* ss, int nss, bool ok, int m, int lane) {
  if (!ok || 4 * lane >= nss) return make_float4(0.f, 0.f, 0.f, 0.f);
  return *(const float4*)(ss + (size_t)m * nss + 4 * lane);
}

__device__ __forceinline__ float norm_rstd(const float* ss, int nss, int K, float eps, bool ok, int m, int lane,
                                           float4 v) {
  float s = ((v.x + v.y) + v.z) + v.w;
  if (ok)
    for (int p = 256 + lane; p < nss; p += 64) s += ss[(size_t)m * nss + p];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
  return 1.0f / sqrtf(s / (float)K + eps);
}

// Packed weight tiles.  A bf16 GEMM weight [N, K] is stored as tiles of 16
// rows (output columns) x 64 K-elements, 1024 elements = 2 KB each, the tiles
// of one row tile consecutive in K.  Inside a tile, element (row c, k) with
// k = 16g + 8h + j (g < 4, h < 2, j < 8) sits at h*512 + (16g + c)*8 + j: lane
// l = 16g + c of a wave reads its MFMA B fragment for K-step h as the 16 bytes
// at h*512 + 8l, so each load instruction of a wave reads 1 KB contiguous.
// The gate and up matrices of a SwiGLU are interleaved tile by tile (gate
// chunk s, up chunk s, gate chunk s+1, ...) so one wave streams one region.
// A dense gate/up weight may use narrower tiles of w < 16 rows (element at
// h*32w + (wg + c)*8 + j, 64w elements per tile) so that its tile count
// spreads evenly over the compute units (swiglu_tile_width); lanes c >= w
// then re-read row w-1 and their MFMA output columns are discarded.
constexpr int PACK_TILE = 1024;   // elements per packed tile

// Fragment order of a GEMM input (bf16 [rows, K]): the packed tile layout
// above with the 16 rows of each row tile in the place of a weight tile's 16
// columns: element (m, k) of chunk k/64 of row tile m/16 at the slot where
// lane 16g + m%16 reads it for K-step h (k%64 = 16g + 8h + j).  A GEMM then
// reads each chunk of its A tile as two 1 KB loads, 8 whole cache lines each,
// where the row-major A touches 16 lines per load instruction.  Producers in
// passes of several rows write this copy next to the row-major one.
__device__ __forceinline__ size_t frag_index(int m, int k, int K) {
  const int q = k & 63;
  return (((size_t)(m >> 4) * (size_t)(K >> 6) + (size_t)(k >> 6)) << 10) + (((q >> 3) & 1) << 9) +
         ((((q >> 4) << 4) + (m & 15)) << 3) + (q & 7);
}

// One wave's share of a 16-row x (NW x 16)-column MFMA tile: the K-chunks
// c0, c0 + step, c0 + 2 step, ... below c1, 64 elements each, accumulated in
// that order.  In each chunk lane group g (lane/16) reads 32 contiguous bytes
// (elements 16g..16g+15) of its A row; the chunk is two MFMA K-steps, the
// first over elements 16g..16g+7 of every group, the second over
// 16g+8..16g+15 (A and B permuted alike).
// xr: this lane's A row at element 16g (xs = 64, xh = 8), or, for an A tile
// in fragment order, at 8*lane (xs = 1024, xh = 512); wr[j]: packed tile j of
// this workgroup at chunk 0 plus 8*lane; consecutive chunks of a tile are NW
// tiles apart (interleaved pairs).  U chunks of loads are issued before their
// MFMAs; weights are read with nontemporal loads (read once per pass).
// CS: elements between consecutive chunks of one weight stream (NW tiles
// interleaved: NW * TE; independent tiles: TE).  TE: elements of one packed
// tile (PACK_TILE, or 64 * width for the narrow gate/up tiles).
template <int NW, bool NT, int U, int CS = NW * PACK_TILE, int TE = PACK_TILE>
__device__ __forceinline__ void mfma_stream(const uint16_t* xr, bool xok, const uint16_t* const* wr, int c0, int c1,
                                            f32x4* acc, int step = 1, int xs = 64, int xh = 8) {
  const uint4 zero = {0u, 0u, 0u, 0u};
  auto ldw = [](const uint16_t* p) { return NT ? ld16_nt(p) : ld16(p); };
  const int n = c1 > c0 ? (c1 - c0 + step - 1) / step : 0;
  int i = 0;
  for (; i + U <= n; i += U) {
    uint4 xa[U][2], wb[NW][U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t s = (size_t)c0 + (size_t)(i + u) * step;
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        wb[j][u][0] = ldw(wr[j] + s * CS);
        wb[j][u][1] = ldw(wr[j] + s * CS + TE / 2);
      }
      xa[u][0] = xok ? ld16(xr + s * xs) : zero;
      xa[u][1] = xok ? ld16(xr + s * xs + xh) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < NW; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[u][h]),
                                                           __builtin_bit_cast(bf16x8, wb[j][u][h]), acc[j], 0, 0, 0);
  }
  for (; i < n; ++i) {
    const size_t s = (size_t)c0 + (size_t)i * step;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 xa = xok ? ld16(xr + s * xs + xh * h) : zero;
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const uint4 wb = ldw(wr[j] + s * CS + h * (TE / 2));
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                         __builtin_bit_cast(bf16x8, wb), acc[j], 0, 0, 0);
      }
    }
  }
}

// As mfma_stream for MT 16-row tiles sharing every weight fragment.
template <int NW, int MT, int CS = NW * PACK_TILE, int TE = PACK_TILE>
__device__ __forceinline__ void mfma_stream_mt(const uint16_t* const* xr, const bool* xok, const uint16_t* const* wr,
                                               int c0, int c1, f32x4 (*acc)[NW]) {
  const uint4 zero = {0u, 0u, 0u, 0u};
  for (int s = c0; s < c1; ++s) {
    uint4 wb[NW][2], xa[MT][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < NW; ++j) wb[j][h] = ld16(wr[j] + (size_t)s * CS + h * (TE / 2));
#pragma unroll
      for (int r = 0; r < MT; ++r) xa[r][h] = xok[r] ? ld16(xr[r] + (size_t)s * 64 + 8 * h) : zero;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int j = 0; j < NW; ++j)
          acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[r][h]),
                                                              __builtin_bit_cast(bf16x8, wb[j][h]), acc[r][j], 0, 0, 0);
  }
}

}  // namespace ssd
