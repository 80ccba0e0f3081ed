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

// MFMA weight-streaming GEMM tile step count issued ahead of their MFMAs
constexpr int GEMM_U = 8;

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *(const uint4*)p; }

// One wave's share of a 16-row x (NW x 16)-column MFMA tile: K-steps
// [s0, s1) of 32 elements, accumulated in order.  xr: this lane's A row at its
// 8-element K group (A rows past the valid ones load zeros); wr[j]: this
// lane's weight row of tile j at the same K group.
template <int NW>
__device__ __forceinline__ void mfma_stream(const uint16_t* xr, bool xok, const uint16_t* const* wr, int s0, int s1,
                                            f32x4* acc) {
  const uint4 zero = {0u, 0u, 0u, 0u};
  int s = s0;
  for (; s + GEMM_U <= s1; s += GEMM_U) {
    uint4 xa[GEMM_U], wb[NW][GEMM_U];
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
#pragma unroll
      for (int j = 0; j < NW; ++j) wb[j][u] = ld16(wr[j] + (size_t)(s + u) * 32);
      xa[u] = xok ? ld16(xr + (size_t)(s + u) * 32) : zero;
    }
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u)
#pragma unroll
      for (int j = 0; j < NW; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[u]),
                                                         __builtin_bit_cast(bf16x8, wb[j][u]), acc[j], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    const uint4 xa = xok ? ld16(xr + (size_t)s * 32) : zero;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const uint4 wb = ld16(wr[j] + (size_t)s * 32);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                       __builtin_bit_cast(bf16x8, wb), acc[j], 0, 0, 0);
    }
  }
}

// As mfma_stream for MT 16-row tiles sharing every weight fragment.
template <int NW, int MT>
__device__ __forceinline__ void mfma_stream_mt(const uint16_t* const* xr, const bool* xok, const uint16_t* const* wr,
                                               int s0, int s1, f32x4 (*acc)[NW]) {
  constexpr int U = 4;
  const uint4 zero = {0u, 0u, 0u, 0u};
  int s = s0;
  for (; s + U <= s1; s += U) {
    uint4 xa[MT][U], wb[NW][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < NW; ++j) wb[j][u] = ld16(wr[j] + (size_t)(s + u) * 32);
#pragma unroll
      for (int r = 0; r < MT; ++r) xa[r][u] = xok[r] ? ld16(xr[r] + (size_t)(s + u) * 32) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int j = 0; j < NW; ++j)
          acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[r][u]),
                                                              __builtin_bit_cast(bf16x8, wb[j][u]), acc[r][j], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    uint4 wb[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) wb[j] = ld16(wr[j] + (size_t)s * 32);
#pragma unroll
    for (int r = 0; r < MT; ++r) {
      const uint4 xa = xok[r] ? ld16(xr[r] + (size_t)s * 32) : zero;
#pragma unroll
      for (int j = 0; j < NW; ++j)
        acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                            __builtin_bit_cast(bf16x8, wb[j]), acc[r][j], 0, 0, 0);
    }
  }
}

}  // namespace ssd
