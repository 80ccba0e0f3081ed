// gfx950 (CDNA4) GEMMs of the greedy self-speculative decode step: the bf16
// weight-streaming GEMM on MFMA with its fused epilogues (QKV + RoPE + KV
// append, residual + folded-norm outputs, SwiGLU, logits + argmax partials),
// the load-time weight packing, and the float32 GEMM of small float32 models.
//
// Every reduction has an order fixed by the shape and by the row's own data
// only, never by the number of rows in the pass (see kernels.hip).
#include "device.h"

// Build-time tuning of the decode GEMMs: load-batch depth in 64-element
// chunks (U1 one-matrix, U2 gate/up with tiles that split evenly over the
// CUs, else 1; the batch depth does not change the accumulation order) and waves per workgroup (gate/up; other
// GEMMs with fewer than 1024 column tiles; wider GEMMs such as the LM head).
#ifndef SSD_GEMM_U1
#define SSD_GEMM_U1 4
#endif
#ifndef SSD_GEMM_U2
#define SSD_GEMM_U2 2
#endif
#ifndef SSD_GEMM_U1_LONGK   // one-matrix GEMMs with K >= 8192 (the FFN down projection)
#define SSD_GEMM_U1_LONGK 2
#endif
#ifndef SSD_GEMM_UW         // GEMMs with >= 1024 column tiles (the LM head)
#define SSD_GEMM_UW 2
#endif
#ifndef SSD_GEMM_U_TPW4     // 4-tile workgroups (the LM head of passes wider than 8 rows):
#define SSD_GEMM_U_TPW4 1   // 84 VGPRs, two workgroups per CU (two chunks: 134, one per CU;
#endif                      // 16 rows: Qwen3-8B head 230.9 -> 217.6 us, Llama-8B 188.6 -> 181.9)
#ifndef SSD_MT_KW            // waves (K ranges) of the multi-row-tile kernel
#define SSD_MT_KW 4
#endif
#ifndef SSD_MT_MT            // 16-row tiles per workgroup of the multi-row-tile kernel
#define SSD_MT_MT 4
#endif
#ifndef SSD_TPW_MIN_M        // tile groups only for passes wider than this
#define SSD_TPW_MIN_M 8
#endif
#ifndef SSD_TPW_MIN_WG       // ... and only where at least this many workgroups remain
#define SSD_TPW_MIN_WG 256
#endif
#ifndef SSD_KW_SWIGLU
#define SSD_KW_SWIGLU 8
#endif
#ifndef SSD_KW_NARROW
#define SSD_KW_NARROW 8
#endif
#ifndef SSD_KW_LONGK_NARROW  // waves (one 64-element chunk per load batch) of K >= 8192 GEMMs in narrow tiles
#define SSD_KW_LONGK_NARROW 16
#endif
#ifndef SSD_TILE_WG_MIN      // long-pass tile kernel: fewest workgroups a wider column group may leave
#define SSD_TILE_WG_MIN 512
#endif
#ifndef SSD_TILE_P1          // long-pass tile kernel: chunks in flight per wave x weight streams
#define SSD_TILE_P1 8
#endif
#ifndef SSD_TILE_PA          // long-pass tile kernel: A chunks in flight per thread
#define SSD_TILE_PA 4
#endif
#ifndef SSD_TILE_MT          // long-pass tile kernel: 16-row tiles per workgroup (even)
#define SSD_TILE_MT 4
#endif
#ifndef SSD_TILE_PB4         // long-pass tile kernel: weight chunks in flight with 4 streams per wave
#define SSD_TILE_PB4 2
#endif
#ifndef SSD_TILE_WPE         // long-pass tile kernel: waves per SIMD the register allocation aims at
#define SSD_TILE_WPE 2
#endif
#ifndef SSD_KW_WIDE
#define SSD_KW_WIDE 8
#endif


namespace ssd {

// ---------------------------------------------------------------------------
// GEMM epilogues
// ---------------------------------------------------------------------------

template <typename E>
__device__ __forceinline__ void epi_single(const GemmArgs& a, int epi, int m, int n, float v) {
  if (epi == EPI_F32) {
    a.y[(size_t)m * a.ldy + n] = v;
  } else if (epi == EPI_LOGITS) {
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
  const E v = fromf<E>(s * u);
  ((E*)a.out)[(size_t)m * a.ldo + n] = v;
  if (sizeof(E) == 2 && a.out_p) ((E*)a.out_p)[frag_index(m, n, a.N)] = v;
}

// (v0, v1) are dims (i, i + hd/2) of output head `head` of [q | k | v]
template <typename E>
__device__ __forceinline__ void epi_qkv_pair(const GemmArgs& a, int base, int m, int head, int i, float v0, float v1) {
  const int half = a.hd >> 1;
  const int pos = base + m;
  if (head < a.hq + a.hkv) {
    const float c = a.cos_t[(size_t)pos * half + i], s = a.sin_t[(size_t)pos * half + i];
    const float o0 = v0 * c - v1 * s, o1 = v1 * c + v0 * s;
    E* dst = head < a.hq ? (E*)a.q + (size_t)m * a.hq * a.hd + (size_t)head * a.hd
                         : (E*)a.kc + ((size_t)(head - a.hq) * a.max_ctx + pos) * a.hd;
    dst[i] = fromf<E>(o0);
    dst[i + half] = fromf<E>(o1);
  } else {   // V cache: [kv head][dim][position]
    E* dst = (E*)a.vc + (size_t)(head - a.hq - a.hkv) * a.hd * a.max_ctx + pos;
    dst[(size_t)i * a.max_ctx] = fromf<E>(v0);
    dst[(size_t)(i + half) * a.max_ctx] = fromf<E>(v1);
  }
}

// as epi_qkv_pair for a q or k head, with the rotary cos/sin already loaded
template <typename E>
__device__ __forceinline__ void epi_qkv_rot(const GemmArgs& a, int base, int m, int head, int i, float v0, float v1,
                                            float c, float s) {
  const int half = a.hd >> 1;
  const int pos = base + m;
  const float o0 = v0 * c - v1 * s, o1 = v1 * c + v0 * s;
  E* dst = head < a.hq ? (E*)a.q + (size_t)m * a.hq * a.hd + (size_t)head * a.hd
                       : (E*)a.kc + ((size_t)(head - a.hq) * a.max_ctx + pos) * a.hd;
  dst[i] = fromf<E>(o0);
  dst[i + half] = fromf<E>(o1);
}

template <typename E>
__device__ __forceinline__ void epi_v_single(const GemmArgs& a, int base, int m, int vh, int dim, float v) {
  const int pos = base + m;
  ((E*)a.vc)[((size_t)vh * a.hd + dim) * a.max_ctx + pos] = fromf<E>(v);   // [kv head][dim][position]
}

// New residual value xv of row m, column n of column tile tt (xv = 0 where
// ok is false: rows past M, lanes past a narrow tile): stores it, its bf16
// tap and the next GEMM's input bf16(xv * gain), and the tile's sum of
// squares (a butterfly over the 16 lanes of the tile; every lane of the wave
// must call this, lane c == 0 writes).
__device__ __forceinline__ void epi_resid_fold(const GemmArgs& a, int m, int n, int tt, int ntiles, int c, bool ok,
                                               float xv) {
  float sq = xv * xv;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o);
  if (ok) {
    const uint16_t xg = f2bf(xv * bf2f(((const uint16_t*)a.gain_next)[n]));
    a.y[(size_t)m * a.ldy + n] = xv;
    if (a.tap) ((uint16_t*)a.tap)[(size_t)m * a.ldtap + n] = f2bf(xv);
    if (a.tap_p) ((uint16_t*)a.tap_p)[frag_index(m, a.tap_col + n, a.ldtap)] = f2bf(xv);
    ((uint16_t*)a.xg_out)[(size_t)m * a.ldy + n] = xg;
    if (a.xg_out_p) ((uint16_t*)a.xg_out_p)[frag_index(m, n, a.N)] = xg;
    if (c == 0) a.ss_out[(size_t)m * ntiles + tt] = sq;
  }
}

// Workgroup -> (column group bx, row block by, column groups gx) of a GEMM
// launch.  A 1-D launch of remap_gx x remap_rb workgroups (set by the
// launcher) maps the row blocks sharing a column group's weights to one XCD
// (workgroups go to the 8 XCDs in turn), dispatched one after another, so
// that XCD's L2 serves the weight tiles to all of them; the mapping never
// changes what a workgroup computes.
struct BlockPos {
  int bx, by, gx;
};
template <bool MAY_REMAP>   // false: launches that never come as the 1-D launch
__device__ __forceinline__ BlockPos block_pos(const GemmArgs& a) {
  if (MAY_REMAP && a.remap_gx > 0) {
    const int L = blockIdx.x, q = L >> 3;
    return BlockPos{(q / a.remap_rb) * 8 + (L & 7), q % a.remap_rb, a.remap_gx};
  }
  return BlockPos{(int)blockIdx.x, (int)blockIdx.y, (int)gridDim.x};
}

// ---------------------------------------------------------------------------
// bf16 skinny GEMM on MFMA 16x16x32 (weight streaming)
//
// Y[M,N] = X[M,K] . W[N,K]^T, M padded to 16-row tiles (grid.y).  A workgroup
// of KW waves owns NW 16-column tiles (NW = 2: the gate and up tiles of the
// same columns); the waves split K into KW contiguous ranges, each
// accumulating its MFMA K-steps in order, and the ranges are added in wave
// order through LDS.  KW and the load-batch depth depend on the shape only,
// so the per-element arithmetic is a function of (shape, row data).  Weights
// come from the packed tile layout (device.h): each wave load instruction
// reads 1 KB contiguous, nontemporal, U 64-element chunks per batch.
//
// MFMA 16x16x32 bf16 lane layout: A row = lane%16, B column = lane%16, both
// with the same 8-element K group lane/16; D: column lane%16, rows
// 4*(lane/16) .. +3.
// ---------------------------------------------------------------------------


__device__ __forceinline__ float4 ss_part(const GemmArgs& a, int m, bool row_ok, int lane) {
  return norm_part(a.ss_in, a.nss, row_ok && m < a.M, m, lane);
}

__device__ __forceinline__ float ss_rstd(const GemmArgs& a, int m, bool row_ok, int lane, float4 v) {
  return norm_rstd(a.ss_in, a.nss, a.K, a.eps, row_ok && m < a.M, m, lane, v);
}

// TPW: independent 16-column tiles per workgroup (one-matrix GEMMs of wide
// passes), sharing every A fragment.  Each tile's MFMA sequence, K split and
// reduction order are those of a one-tile workgroup, so TPW never changes a
// result; it only cuts the A-operand reads from L2.
//
// TW: rows per packed tile (16; 14 for narrow gate/up tiles, 12 for narrow
// QKV tiles; lanes c >= TW compute discarded columns).  A column's
// arithmetic does not depend on TW.
template <int EPI, int NW, int KW, int MT, int U, int TPW, int TW = 16>
__global__ __launch_bounds__(64 * KW) void gemm_bf16_kernel(GemmArgs a) {
  static_assert(TPW == 1 || NW == 1 || MT > 1, "gate/up tile groups are for multi-row-tile launches");
  static_assert(TW == 16 || (EPI == EPI_SWIGLU && TW == 14) || (EPI == EPI_QKV && TW == 12) ||
                    (EPI == EPI_RESID && (TW == 10 || TW == 8)),
                "tile width");
  constexpr int NS = NW * TPW;                               // weight streams
  constexpr int TE = TW * 64;                                // elements per packed tile
  constexpr int CS = NW > 1 ? NW * TE : TE;                  // chunk stride of a stream
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, kg = lane >> 4;
  // workgroup -> (column group bx, row block by); multi-row-tile launches may
  // come as the XCD-aware 1-D launch (block_pos)
  const BlockPos bp = block_pos<(MT > 1)>(a);
  const int bx = bp.bx, by = bp.by;
  const int t0 = bx * TPW;                                   // first column tile
  const int ntiles = bp.gx * TPW;
  const uint16_t* xr[MT];
  bool av_ok[MT];
#pragma unroll
  for (int r = 0; r < MT; ++r) {
    const int am = (by * MT + r) * 16 + c;
    av_ok[r] = am < a.M;
    xr[r] = (const uint16_t*)a.X + (size_t)(av_ok[r] ? am : 0) * a.ldx + kg * 16;
  }
  const int S = a.K >> 6;   // 64-element chunks
  // an A tile in fragment order (decode passes of several rows): each chunk
  // is two 1 KB loads (the same values, so the same results)
  const bool xfrag = MT == 1 && a.Xp != nullptr;
  if (xfrag) xr[0] = (const uint16_t*)a.Xp + ((size_t)by * S << 10) + 8 * lane;
  const int xs = xfrag ? 1024 : 64, xh = xfrag ? 512 : 8;
  // packed weight tiles: gate/up interleaved when NW = 2, else TPW tiles
  // stream j: matrix j % NW of column tile t0 + j / NW
  const uint16_t* wr[NS];
  const int lo = (TW * kg + min(c, TW - 1)) * 8;             // this lane's 16 bytes in a tile half
#pragma unroll
  for (int j = 0; j < NS; ++j)
    wr[j] = NW > 1 ? (const uint16_t*)a.W0 + ((size_t)(t0 + j / NW) * S * NW + j % NW) * TE + lo
                   : (const uint16_t*)a.W0 + (size_t)(t0 + j) * S * TE + lo;
  int head[TPW], dim[TPW], kind[TPW];   // QKV output column of this lane (qkv_col_map)
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    head[j] = dim[j] = 0;
    kind[j] = 1;
    if (EPI == EPI_QKV) {
      const QkvCol q = qkv_col_map(TW, t0 + j, c, a.hq, a.hkv, a.hd);
      head[j] = q.head;
      dim[j] = q.dim;
      kind[j] = q.kind;
    }
  }

  // K split over the waves: in the LM head and the o projection (one-tile
  // launches) wave w takes chunks w, w + KW, ..., so the waves of a
  // workgroup read adjacent chunks at each step (measured faster there:
  // LM head at 16 rows 188 -> 181 us, o at 6 rows 8.5 -> 8.1 us); elsewhere
  // each wave takes the contiguous range [s0, s1).  The choice depends on
  // the epilogue and K only, never on the pass width.
  const bool kil = MT == 1 && (EPI == EPI_LOGITS || (EPI == EPI_RESID && a.K < 8192));
  const int s0 = kil ? wave : (S * wave) / KW, s1 = kil ? S : (S * (wave + 1)) / KW;
  const int kst = kil ? KW : 1;

  // Epilogue split: in one-tile-row launches wave e < 4 finishes accumulator
  // element e (rows 4kg + e) of every lane, so up to four rows' epilogues run
  // side by side; other launches finish on wave 0.  ep(i): element i is this
  // wave's.
  constexpr bool SPLIT = MT == 1 && KW >= 4;
  auto ep = [&](int i) { return SPLIT ? i == wave : wave == 0; };

  // Epilogue inputs fetched before the weight stream so that their latency
  // hides behind it: the position base (QKV) and, for one-tile-row launches,
  // the residual entries this wave will update.
  const int base = EPI == EPI_QKV ? a.state[0] + a.pos_off : 0;
  float yv[TPW][4];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) yv[j][i] = 0.f;
  if (EPI == EPI_RESID && MT == 1) {
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = by * 16 + 4 * kg + i;
        if (ep(i) && m < a.M && c < TW) yv[j][i] = a.y[(size_t)m * a.ldy + (t0 + j) * TW + c];
      }
  }

  // folded RMSNorm: wave w owns tile rows w, w + KW, ...  One-tile launches
  // load the rows' sum-of-squares partials before the weight stream so the
  // loads overlap it; multi-tile launches load them afterwards.
  constexpr int RPW = (16 * MT + KW - 1) / KW;   // rows per wave
  constexpr int RPRE = MT == 1 ? RPW : 1;
  const bool fold = a.ss_in != nullptr;
  float4 ssv[RPRE];
  if (MT == 1 && fold) {
#pragma unroll
    for (int r = 0; r < RPRE; ++r) ssv[r] = ss_part(a, by * 16 + wave + r * KW, r * KW + wave < 16, lane);
  }
  f32x4 acc[MT][NS];
#pragma unroll
  for (int r = 0; r < MT; ++r)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float rc[TPW][4], rsn[TPW][4];   // RoPE cos/sin (QKV)
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) rc[j][i] = rsn[j][i] = 0.f;
  if (MT == 1 && EPI == EPI_QKV) {
    // first load batch, then the rotary table entries of this wave's
    // epilogue rows (they need the position), then the rest of the K range
    const int sm = min(s0 + U * kst, s1);
    mfma_stream<NS, true, U, CS, TE>(xr[0], av_ok[0], wr, s0, sm, acc[0], kst, xs, xh);
    {
      const int half = a.hd >> 1;
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        if (kind[j] != 0) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = by * 16 + 4 * kg + i;
          if (ep(i) && m < a.M) {
            rc[j][i] = a.cos_t[(size_t)(base + m) * half + dim[j]];
            rsn[j][i] = a.sin_t[(size_t)(base + m) * half + dim[j]];
          }
        }
      }
    }
    mfma_stream<NS, true, U, CS, TE>(xr[0], av_ok[0], wr, sm, s1, acc[0], kst, xs, xh);
  } else if (MT == 1) {
    mfma_stream<NS, true, U, CS, TE>(xr[0], av_ok[0], wr, s0, s1, acc[0], kst, xs, xh);
  }
  else mfma_stream_mt<NS, MT, CS, TE>(xr, av_ok, wr, s0, s1, acc);

  __shared__ f32x4 red[SPLIT ? KW : KW - 1][MT][NS][64];
  __shared__ float rs[16 * MT];
  if (fold) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = r * KW + wave;
      const int m = by * 16 * MT + row;
      const float4 v = MT == 1 ? ssv[r < RPRE ? r : 0] : ss_part(a, m, row < 16 * MT, lane);
      const float f = ss_rstd(a, m, row < 16 * MT, lane, v);
      if (lane == 0 && row < 16 * MT) rs[row] = f;
    }
  }
  if (SPLIT) {
    // every wave's partial sums to LDS; wave e < 4 adds element e of them in
    // wave order (the order of the unsplit reduction, so the same sums)
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
      for (int j = 0; j < NS; ++j) red[wave][r][j][lane] = acc[r][j];
    __syncthreads();
    if (wave >= 4) return;
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        float v = ((const float*)&red[0][r][j][lane])[wave];
#pragma unroll
        for (int w = 1; w < KW; ++w) v += ((const float*)&red[w][r][j][lane])[wave];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[r][j][i] = i == wave ? v : acc[r][j][i];
      }
  } else {
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int j = 0; j < NS; ++j) red[wave - 1][r][j][lane] = acc[r][j];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < KW - 1; ++w)
#pragma unroll
      for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[r][j] = acc[r][j] + red[w][r][j][lane];
  }
  if (fold) {
    // rows of this lane's accumulators: 4*kg + i of each 16-row tile
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = rs[r * 16 + 4 * kg + i];
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[r][j][i] *= f;
      }
  }

#pragma unroll
  for (int r = 0; r < MT; ++r) {
    const int mt = by * MT + r;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!ep(i)) continue;
          const int m = mt * 16 + 4 * kg + i;
          if (m < a.M && c < TW)
            epi_swiglu<uint16_t>(a, m, (t0 + jt) * TW + c, acc[r][jt * NW][i], acc[r][jt * NW + NW - 1][i]);
        }
      continue;
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int tt = t0 + j;   // column tile
      if (EPI == EPI_QKV) {
        // a pair's second element sits TW/2 lanes up (same 16-lane group)
        float part[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) part[i] = __shfl(acc[r][j][i], (lane + TW / 2) & 63);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mt * 16 + 4 * kg + i;
          if (!ep(i) || m >= a.M) continue;
          if (kind[j] == 0) {
            if (MT == 1)
              epi_qkv_rot<uint16_t>(a, base, m, head[j], dim[j], acc[r][j][i], part[i], rc[j][i], rsn[j][i]);
            else epi_qkv_pair<uint16_t>(a, base, m, head[j], dim[j], acc[r][j][i], part[i]);
          } else if (kind[j] == 2) {
            epi_v_single<uint16_t>(a, base, m, head[j] - a.hq - a.hkv, dim[j], acc[r][j][i]);
          }
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!ep(i)) continue;
        const int m = mt * 16 + 4 * kg + i;
        const int n = tt * TW + c;   // lanes c >= TW (narrow residual tiles) write nothing
        if (EPI == EPI_LOGITS) {
          // (max, lowest index) over this tile's 16 columns, fixed butterfly
          float bv = acc[r][j][i];
          int bi = n;
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            const float ov = __shfl_xor(bv, o);
            const int oi = __shfl_xor(bi, o);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
          }
          if (m < a.M && c == 0) {
            a.amax_v[(size_t)m * ntiles + tt] = bv;
            a.amax_i[(size_t)m * ntiles + tt] = bi;
          }
        }
        if (EPI == EPI_RESID && a.ss_out) {
          // new residual, its sum of squares over this tile's 16 columns and
          // bf16(x * gain) for the GEMM that consumes it
          const bool ok = m < a.M && c < TW;
          const float xv = ok ? (MT == 1 ? yv[j][i] : a.y[(size_t)m * a.ldy + n]) + acc[r][j][i] : 0.f;
          epi_resid_fold(a, m, n, tt, ntiles, c, ok, xv);
          continue;
        }
        if (m >= a.M || c >= TW) continue;
        if (EPI == EPI_RESID && MT == 1) {
          const float xv = yv[j][i] + acc[r][j][i];
          a.y[(size_t)m * a.ldy + n] = xv;
          if (a.tap) ((uint16_t*)a.tap)[(size_t)m * a.ldtap + n] = f2bf(xv);
          if (a.tap_p) ((uint16_t*)a.tap_p)[frag_index(m, a.tap_col + n, a.ldtap)] = f2bf(xv);
        } else epi_single<uint16_t>(a, EPI, m, n, acc[r][j][i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Layer GEMMs of long passes (prefill chunks, M > 32: QKV + RoPE + KV append,
// gate/up + SwiGLU, o and down + residual) on MFMA 16x16x32 with the A
// operand staged through LDS.
//
// A workgroup of 4 waves owns 16*MT rows and 4 * NTW column tiles; wave w
// owns tiles t0 + w*NTW .. t0 + w*NTW + NTW - 1 (both gate/up streams of
// each) for all the rows.  Every output element accumulates its MFMA K-steps
// in K order over the whole K range: no K split, no cross-wave reduction,
// and nothing depends on M or on the grouping.  Per 64-element K chunk the
// workgroup copies the A block into one of two LDS buffers (one barrier per
// chunk) while each thread keeps the A pieces of the next PA - 1 chunks and
// each wave the weight fragments of the next PB - 1 chunks in flight in
// registers (PB = 8 / streams, at least 2); a wave reads its A fragments from
// LDS once per chunk for all its column tiles and reuses each weight fragment
// for every row tile.  Measured at 256 rows (8B shape) against the
// multi-row-tile kernel: gate/up 209 -> 99 us, down 144 -> 74, QKV 66 -> 46,
// o 51 -> 29.
// ---------------------------------------------------------------------------
constexpr int TILE_WAVES = 4;
constexpr int TILE_MT = SSD_TILE_MT;   // row tiles per workgroup
constexpr int TILE_LDA = 64 + 8;       // LDS row stride of the A block (elements): rows 144 B apart

constexpr int tile_lcm(int x, int y) {
  int a = x, b = y;
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return x / a * y;
}
// ring depths of a wave with ns weight streams, and the unroll that makes
// every ring index static (the K chunks must be a multiple of it)
constexpr int tile_pb(int ns) { return ns >= 4 ? SSD_TILE_PB4 : SSD_TILE_P1 / ns; }
constexpr int tile_unroll(int ns) { return tile_lcm(tile_lcm(SSD_TILE_PA, tile_pb(ns)), 2); }

template <int EPI, int TW, int NTW>
__global__ __launch_bounds__(64 * TILE_WAVES) __attribute__((amdgpu_waves_per_eu(SSD_TILE_WPE)))
void gemm_tile_kernel(GemmArgs a) {
  static_assert(EPI == EPI_QKV || EPI == EPI_SWIGLU || EPI == EPI_RESID, "layer GEMM epilogues");
  constexpr int NW = EPI == EPI_SWIGLU ? 2 : 1;   // gate/up: two interleaved streams per tile
  constexpr int MT = TILE_MT, NS = NW * NTW, TE = TW * 64, CS = NW * TE;
  constexpr int NA = MT / 2;                           // 16-byte A pieces per thread and chunk
  static_assert(MT % 2 == 0, "A block copy");
  constexpr int PB = tile_pb(NS);      // weight chunks in flight per wave
  constexpr int PA = SSD_TILE_PA;      // A chunks in flight (4 * NA registers each)
  constexpr int U = tile_unroll(NS);
  static_assert(PB >= 2 && PA >= 2, "ring depths");
  constexpr int ROWS = 16 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][ROWS * TILE_LDA];
  __shared__ float rs[ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, kg = lane >> 4;
  const BlockPos bp = block_pos<true>(a);           // column group, row block (XCD-aware order)
  const int t0 = (bp.bx * TILE_WAVES + wave) * NTW;   // this wave's first column tile
  const int row0 = bp.by * ROWS;
  const int S = a.K >> 6;

  // weight streams: stream j = matrix j % NW (gate, up) of column tile t0 + j / NW
  const uint16_t* wr[NS];
  const int lo = (TW * kg + min(c, TW - 1)) * 8;
#pragma unroll
  for (int j = 0; j < NS; ++j)
    wr[j] = (const uint16_t*)a.W0 + ((size_t)(t0 + j / NW) * S * NW + j % NW) * TE + lo;

  // A block copy: 16*MT rows x 64 elements = 128*MT pieces of 16 bytes, NA
  // per thread (piece p: row p / 8, elements 8 * (p % 8) ..)
  const uint16_t* ag[NA];
  bool aok[NA];
  int aoff[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int p = tid + 64 * TILE_WAVES * i, r = p >> 3, cc = p & 7;
    aok[i] = row0 + r < a.M;
    ag[i] = (const uint16_t*)a.X + (size_t)(aok[i] ? row0 + r : 0) * a.ldx + cc * 8;
    aoff[i] = r * TILE_LDA + cc * 8;
  }
  const uint4 zero = {0u, 0u, 0u, 0u};
  uint4 areg[PA][NA];
  uint4 wb[PB][NS][2];
  f32x4 acc[MT][NS];
#pragma unroll
  for (int r = 0; r < MT; ++r)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // every load below is unconditional (rows past M read row 0 and are
  // masked to zero, chunk indexes past the end are clamped): branches in the
  // loop would make the compiler drain all loads in flight at each chunk
  unsigned amask[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) amask[i] = aok[i] ? ~0u : 0u;
  auto load_a = [&](uint4 (&ar)[NA], int s) {
#pragma unroll
    for (int i = 0; i < NA; ++i) ar[i] = ld16(ag[i] + (size_t)s * 64);
  };
  auto store_a = [&](int buf, const uint4 (&ar)[NA]) {   // masked here, where the data is due anyway
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const uint4 v = ar[i];
      *(uint4*)(&As[buf][aoff[i]]) = uint4{v.x & amask[i], v.y & amask[i], v.z & amask[i], v.w & amask[i]};
    }
  };
  auto load_w = [&](uint4 (&w)[NS][2], int s) {   // cached loads: the row blocks share the tiles
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) w[j][h] = ld16(wr[j] + (size_t)s * CS + h * (TE / 2));
  };
  // lane (c, kg) of row tile r reads row 16r + c, elements 16kg + 8h .. + 7
  // of the chunk: the MFMA A fragment of K-step h
  auto compute = [&](int buf, const uint4 (&w)[NS][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 af[MT];
#pragma unroll
      for (int r = 0; r < MT; ++r) af[r] = *(const uint4*)(&As[buf][(16 * r + c) * TILE_LDA + 16 * kg + 8 * h]);
#pragma unroll
      for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int j = 0; j < NS; ++j)
          acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[r]),
                                                              __builtin_bit_cast(bf16x8, w[j][h]), acc[r][j], 0, 0, 0);
    }
  };

  // chunk s: A pieces areg[s % PA] -> LDS buffer s & 1, weights wb[s % PB].
  // Iteration s issues the A loads of chunk s + PA - 1 and the weight loads
  // of chunk s + PB - 1 (clamped to the last chunk), computes chunk s and
  // moves chunk s + 1's A pieces into the other LDS buffer (whose chunk s - 1
  // every wave finished before the previous barrier).  The launcher
  // guarantees S % U == 0.
  const int last = S - 1;
#pragma unroll
  for (int u = 0; u < PA - 1; ++u) load_a(areg[u], min(u, last));
#pragma unroll
  for (int u = 0; u < PB - 1; ++u) load_w(wb[u], min(u, last));
  store_a(0, areg[0]);
  __syncthreads();
  for (int s0 = 0; s0 < S; s0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      load_a(areg[(u + PA - 1) % PA], min(s + PA - 1, last));
      load_w(wb[(u + PB - 1) % PB], min(s + PB - 1, last));
      // keep the prefetch loads ahead of this chunk's MFMAs (the scheduler
      // would otherwise sink them towards their uses and wait on them)
      __builtin_amdgcn_sched_barrier(0);
      compute(u & 1, wb[u % PB]);
      store_a((u + 1) & 1, areg[(u + 1) % PA]);
      __syncthreads();
    }
  }

  // folded RMSNorm: wave w finds rstd of rows w, w + 4, ...
  const bool fold = a.ss_in != nullptr;
  if (fold) {
#pragma unroll 1
    for (int r = 0; r < ROWS / TILE_WAVES; ++r) {
      const int row = r * TILE_WAVES + wave, m = row0 + row;
      const float f = ss_rstd(a, m, true, lane, ss_part(a, m, true, lane));
      if (lane == 0) rs[row] = f;
    }
  }
  __syncthreads();
  if (fold) {
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = rs[16 * r + 4 * kg + i];
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[r][j][i] *= f;
      }
  }
  // epilogue: each wave finishes its own column tiles for all its rows
  int head[NTW], dim[NTW], kind[NTW];   // QKV output column of this lane (qkv_col_map)
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    head[j] = dim[j] = 0;
    kind[j] = 1;
    if (EPI == EPI_QKV) {
      const QkvCol q = qkv_col_map(TW, t0 + j, c, a.hq, a.hkv, a.hd);
      head[j] = q.head;
      dim[j] = q.dim;
      kind[j] = q.kind;
    }
  }
  const int base = EPI == EPI_QKV ? a.state[0] + a.pos_off : 0;
  const int ntiles = bp.gx * TILE_WAVES * NTW;
#pragma unroll
  for (int r = 0; r < MT; ++r)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int tt = t0 + j;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = row0 + 16 * r + 4 * kg + i;
          if (m < a.M && c < TW) epi_swiglu<uint16_t>(a, m, tt * TW + c, acc[r][j * NW][i], acc[r][j * NW + 1][i]);
        }
      } else if (EPI == EPI_QKV) {
        // a pair's second element sits TW/2 lanes up (same 16-lane group)
        float part[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) part[i] = __shfl(acc[r][j][i], (lane + TW / 2) & 63);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = row0 + 16 * r + 4 * kg + i;
          if (m >= a.M) continue;
          if (kind[j] == 0) epi_qkv_pair<uint16_t>(a, base, m, head[j], dim[j], acc[r][j][i], part[i]);
          else if (kind[j] == 2) epi_v_single<uint16_t>(a, base, m, head[j] - a.hq - a.hkv, dim[j], acc[r][j][i]);
        }
      } else {   // EPI_RESID
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = row0 + 16 * r + 4 * kg + i;
          const int n = tt * TW + c;
          const bool ok = m < a.M && c < TW;
          if (a.ss_out) {
            const float xv = ok ? a.y[(size_t)m * a.ldy + n] + acc[r][j][i] : 0.f;
            epi_resid_fold(a, m, n, tt, ntiles, c, ok, xv);
          } else if (ok) {
            epi_single<uint16_t>(a, EPI_RESID, m, n, acc[r][j][i]);
          }
        }
      }
    }
}

// ---------------------------------------------------------------------------
// weight packing (load time): one workgroup per packed tile, 16 bytes per thread
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(128) void pack_kernel(PackArgs p) {
  const int t = blockIdx.x, s = blockIdx.y, which = blockIdx.z;
  const int l = threadIdx.x & 63, h = threadIdx.x >> 6, g = l >> 4, c = l & 15;
  const int tw = p.tw ? p.tw : 16;   // rows per tile
  const uint16_t* src;
  size_t row;
  if (c >= tw) return;
  if (p.mode == 1) {
    const QkvCol q = qkv_col_map(tw, t, c, p.hq, p.hkv, p.hd);
    const int head = q.head, dim = q.dim;
    if (head < p.hq) { src = (const uint16_t*)p.src0; row = (size_t)head * p.hd + dim; }
    else if (head < p.hq + p.hkv) { src = (const uint16_t*)p.src1; row = (size_t)(head - p.hq) * p.hd + dim; }
    else { src = (const uint16_t*)p.src2; row = (size_t)(head - p.hq - p.hkv) * p.hd + dim; }
  } else {
    src = (const uint16_t*)(which ? p.src1 : p.src0);
    row = (size_t)t * tw + c;
  }
  const uint4 v = *(const uint4*)(src + row * p.K + (size_t)s * 64 + 16 * g + 8 * h);
  const size_t tile = ((size_t)t * (p.K / 64) + s) * (p.pair ? 2 : 1) + which;
  *(uint4*)((uint16_t*)p.dst + tile * (64 * tw) + h * (32 * tw) + (tw * g + c) * 8) = v;
}

hipError_t launch_pack(const PackArgs& p, hipStream_t s) {
  const int tw = p.tw ? p.tw : 16;
  if (tw < 1 || tw > 16 || (p.mode == 1 && tw != 16 && tw != 12)) return hipErrorInvalidValue;
  if (p.mode == 1 && (tw == 16 ? p.hd % 16 : p.hd % 2)) return hipErrorInvalidValue;
  if (p.N % tw || p.N % 16 || p.K % 64 || p.N <= 0 || p.K <= 0) return hipErrorInvalidValue;
  pack_kernel<<<dim3(p.N / tw, p.K / 64, p.pair ? 2 : 1), 128, 0, s>>>(p);
  return hipGetLastError();
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
      if (EPI == EPI_QKV) epi_qkv_pair<float>(a, a.state[0] + a.pos_off, m, head, i, s0, s1);
      else if (EPI == EPI_SWIGLU) epi_swiglu<float>(a, m, pi, s0, s1);
      else {
        epi_single<float>(a, EPI, m, 2 * pi, s0);
        epi_single<float>(a, EPI, m, 2 * pi + 1, s1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s) {
  const int mt = (a.M + 15) / 16;
  if (dtype) {
    int tiles;
    const int tw = epi == EPI_SWIGLU ? swiglu_tile_width(a.N)   // as packed
                   : epi == EPI_QKV   ? qkv_tile_width(a.hq, a.hkv, a.hd)
                   : epi == EPI_RESID ? resid_tile_width(a.N)
                                      : 16;
    // the folded norm's partials come one per residual tile
    if (epi == EPI_RESID && a.ss_out && a.N % tw != 0) return hipErrorInvalidValue;
    if (epi == EPI_QKV) tiles = (a.hq + 2 * a.hkv) * a.hd / tw;
    else tiles = a.N / tw;
    dim3 grid(tiles, mt);
    const bool wide = tiles >= 1024;   // a function of N only
    // gate/up of long passes (prefill chunks): the LDS-staged tile kernel,
    // 64 rows x 4*ntw column tiles per workgroup, ntw = 2 where that still
    // leaves SSD_TILE_WG_MIN workgroups (the grouping never changes a result)
    // streams per wave: 1, 2 or 4 (gate/up: 2 or 4), any of which the
    // grouping may pick, so the K chunks must suit every ring unroll
    constexpr int tile_u = tile_lcm(tile_lcm(tile_unroll(1), tile_unroll(2)), tile_unroll(4));
    const bool tile_epi = epi == EPI_QKV || epi == EPI_SWIGLU || epi == EPI_RESID;
    if (a.M > 32 && tile_epi && tiles % TILE_WAVES == 0 && (a.K / 64) % tile_u == 0) {
      const int rbt = (a.M + 16 * TILE_MT - 1) / (16 * TILE_MT);
      const int wg_min = a.tile_wg_min > 0 ? a.tile_wg_min : SSD_TILE_WG_MIN;
      int ntw = 1;
      for (int v = epi == EPI_SWIGLU ? 2 : 4; v > 1; v >>= 1)
        if (tiles % (TILE_WAVES * v) == 0 && (tiles / (TILE_WAVES * v)) * rbt >= wg_min) {
          ntw = v;
          break;
        }
      const int gx = tiles / (TILE_WAVES * ntw);
      GemmArgs at = a;
      at.remap_gx = at.remap_rb = 0;
      dim3 g(gx, rbt);
      if (gx % 8 == 0 && rbt > 1) {   // XCD-aware 1-D launch (see gemm_bf16_kernel)
        at.remap_gx = gx;
        at.remap_rb = rbt;
        g = dim3(gx * rbt, 1);
      }
      const dim3 blk(64 * TILE_WAVES);
#define SSD_T(E, TWV)                                                                 \
  {                                                                                   \
    if (ntw == 4) gemm_tile_kernel<E, TWV, E == EPI_SWIGLU ? 2 : 4><<<g, blk, 0, s>>>(at); \
    else if (ntw == 2) gemm_tile_kernel<E, TWV, 2><<<g, blk, 0, s>>>(at);             \
    else gemm_tile_kernel<E, TWV, 1><<<g, blk, 0, s>>>(at);                           \
  }
      if (epi == EPI_SWIGLU) {
        if (tw == 14) SSD_T(EPI_SWIGLU, 14) else SSD_T(EPI_SWIGLU, 16)
      } else if (epi == EPI_QKV) {
        if (tw == 12) SSD_T(EPI_QKV, 12) else SSD_T(EPI_QKV, 16)
      } else {
        if (tw == 10) SSD_T(EPI_RESID, 10) else if (tw == 8) SSD_T(EPI_RESID, 8) else SSD_T(EPI_RESID, 16)
      }
#undef SSD_T
      return hipGetLastError();
    }
    // decode-loop passes (M <= SSD_MAX_BLOCK rows) always take the one-tile
    // kernel, so a row's arithmetic never depends on the pass width; longer
    // passes (prefill chunks) let 4 row tiles share each weight load
    const bool multi = a.M > 32;
    // long passes group column tiles too, so each workgroup reads its 64 A
    // rows once for 2 or 4 tiles, while keeping two workgroups per CU
    const int rb = (a.M + 16 * SSD_MT_MT - 1) / (16 * SSD_MT_MT);
    int tpm = 1;
    if (multi && tiles % 4 == 0 && (tiles / 4) * rb >= 2 * NUM_CU && epi != EPI_SWIGLU) tpm = 4;
    else if (multi && tiles % 2 == 0 && (tiles / 2) * rb >= 2 * NUM_CU) tpm = 2;
    dim3 grid_mt(tiles / tpm, rb);
    GemmArgs am = a;
    am.remap_gx = am.remap_rb = 0;
    if (multi && (tiles / tpm) % 8 == 0 && rb > 1) {   // XCD-aware 1-D launch (see the kernel)
      am.remap_gx = tiles / tpm;
      am.remap_rb = rb;
      grid_mt = dim3((tiles / tpm) * rb, 1);
    }
    // passes wider than 8 rows group 2 or 4 column tiles per workgroup so
    // the A operand is read once for them (results unchanged, see the kernel),
    // but only where at least SSD_TPW_MIN_WG workgroups remain, one per CU:
    // spreading the weight stream over every CU matters more than the A reads
    // (measured at 16 rows: the LM head 250 -> 231 us with 4 tiles, 218 with
    // one-chunk batches, QKV of 512 tiles 13.7 -> 12.1 us with 2; o and down
    // keep their 256 workgroups; at 5-8 rows the grouped LM head is slower,
    // 191 -> 203 us at 6 rows, whatever the batch depth)
    // (never for long-K narrow tiles: their one-tile kernel splits K over
    // more waves, and a row's K split must not depend on the pass width)
    int tpw = 1;
    const bool tpw_ok = a.M > SSD_TPW_MIN_M && !(a.K >= 8192 && tw < 16);
    if (tpw_ok && tiles % 4 == 0 && tiles / 4 >= SSD_TPW_MIN_WG) tpw = 4;
    else if (tpw_ok && tiles % 2 == 0 && tiles / 2 >= SSD_TPW_MIN_WG) tpw = 2;
#define SSD_G1(E, KWN, UN, TWV)                                                                         \
  if (multi) {                                                                                           \
    if (tpm == 4) gemm_bf16_kernel<E, 1, SSD_MT_KW, SSD_MT_MT, 1, 4, TWV><<<grid_mt, 64 * SSD_MT_KW, 0, s>>>(am); \
    else if (tpm == 2) gemm_bf16_kernel<E, 1, SSD_MT_KW, SSD_MT_MT, 1, 2, TWV><<<grid_mt, 64 * SSD_MT_KW, 0, s>>>(am); \
    else gemm_bf16_kernel<E, 1, SSD_MT_KW, SSD_MT_MT, 1, 1, TWV><<<grid_mt, 64 * SSD_MT_KW, 0, s>>>(am);   \
  }                                                                                                      \
  else if (tpw == 4) {                                                                                   \
    const dim3 g4(tiles / 4, mt);                                                                        \
    if (wide) gemm_bf16_kernel<E, 1, SSD_KW_WIDE, 1, SSD_GEMM_U_TPW4, 4, TWV><<<g4, 64 * SSD_KW_WIDE, 0, s>>>(a); \
    else gemm_bf16_kernel<E, 1, KWN, 1, SSD_GEMM_U_TPW4, 4, TWV><<<g4, 64 * KWN, 0, s>>>(a);              \
  } else if (tpw == 2) {                                                                                 \
    const dim3 g2(tiles / 2, mt);                                                                        \
    if (wide) gemm_bf16_kernel<E, 1, SSD_KW_WIDE, 1, 2, 2, TWV><<<g2, 64 * SSD_KW_WIDE, 0, s>>>(a);      \
    else gemm_bf16_kernel<E, 1, KWN, 1, 2, 2, TWV><<<g2, 64 * KWN, 0, s>>>(a);                           \
  } else if (wide) gemm_bf16_kernel<E, 1, SSD_KW_WIDE, 1, SSD_GEMM_UW, 1, TWV><<<grid, 64 * SSD_KW_WIDE, 0, s>>>(a); \
  else if (a.K >= 8192) {                                                                               \
    if constexpr (TWV < 16)                                                                              \
      gemm_bf16_kernel<E, 1, SSD_KW_LONGK_NARROW, 1, 1, 1, TWV><<<grid, 64 * SSD_KW_LONGK_NARROW, 0, s>>>(a); \
    else gemm_bf16_kernel<E, 1, KWN, 1, SSD_GEMM_U1_LONGK, 1, TWV><<<grid, 64 * KWN, 0, s>>>(a);          \
  }                                                                                                      \
  else gemm_bf16_kernel<E, 1, KWN, 1, UN, 1, TWV><<<grid, 64 * KWN, 0, s>>>(a);
    switch (epi) {
      case EPI_F32: SSD_G1(EPI_F32, SSD_KW_NARROW, SSD_GEMM_U1, 16) break;
      case EPI_LOGITS: SSD_G1(EPI_LOGITS, SSD_KW_NARROW, SSD_GEMM_U1, 16) break;
      case EPI_RESID:
        if (tw == 10) { SSD_G1(EPI_RESID, SSD_KW_NARROW, SSD_GEMM_U1, 10) }
        else if (tw == 8) { SSD_G1(EPI_RESID, SSD_KW_NARROW, SSD_GEMM_U1, 8) }
        else { SSD_G1(EPI_RESID, SSD_KW_NARROW, SSD_GEMM_U1, 16) }
        break;
      case EPI_QKV:
        if (tw == 12) { SSD_G1(EPI_QKV, SSD_KW_NARROW, SSD_GEMM_U1, 12) }
        else { SSD_G1(EPI_QKV, SSD_KW_NARROW, SSD_GEMM_U1, 16) }
        break;
      case EPI_STORE: SSD_G1(EPI_STORE, SSD_KW_NARROW, SSD_GEMM_U1, 16) break;
      case EPI_SWIGLU: {
        // Load batches of the one-tile kernel: SSD_GEMM_U2 chunks where the
        // tiles split evenly over the CUs, else one, so that every workgroup
        // is resident at once (58 instead of 90 VGPRs) and no CU runs a last
        // round alone (measured: 608 tiles of the Qwen3-4B shape 20.3 ->
        // 19.2 us; 768 and 1024 tiles faster with two, 33.9 -> 33.0 and
        // 37.1 -> 36.4 us).  The batch depth never changes a result.
        const bool u1 = tiles % NUM_CU != 0;
        if (tw == 14) {
          if (multi && tpm == 2) gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_MT_KW, SSD_MT_MT, 1, 2, 14><<<grid_mt, 64 * SSD_MT_KW, 0, s>>>(am);
          else if (multi) gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_MT_KW, SSD_MT_MT, 1, 1, 14><<<grid_mt, 64 * SSD_MT_KW, 0, s>>>(am);
          else if (u1) gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_KW_SWIGLU, 1, 1, 1, 14><<<grid, 64 * SSD_KW_SWIGLU, 0, s>>>(a);
          else gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_KW_SWIGLU, 1, SSD_GEMM_U2, 1, 14><<<grid, 64 * SSD_KW_SWIGLU, 0, s>>>(a);
        } else if (multi && tpm == 2) gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_MT_KW, SSD_MT_MT, 1, 2><<<grid_mt, 64 * SSD_MT_KW, 0, s>>>(am);
        else if (multi) gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_MT_KW, SSD_MT_MT, 1, 1><<<grid_mt, 64 * SSD_MT_KW, 0, s>>>(am);
        else if (wide && u1) gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_KW_WIDE, 1, 1, 1><<<grid, 64 * SSD_KW_WIDE, 0, s>>>(a);
        else if (wide) gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_KW_WIDE, 1, SSD_GEMM_U2, 1><<<grid, 64 * SSD_KW_WIDE, 0, s>>>(a);
        else if (u1) gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_KW_SWIGLU, 1, 1, 1><<<grid, 64 * SSD_KW_SWIGLU, 0, s>>>(a);
        else gemm_bf16_kernel<EPI_SWIGLU, 2, SSD_KW_SWIGLU, 1, SSD_GEMM_U2, 1><<<grid, 64 * SSD_KW_SWIGLU, 0, s>>>(a);
        break;
      }
      default: return hipErrorInvalidValue;
    }
#undef SSD_G1
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

}  // namespace ssd
