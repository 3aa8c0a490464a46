// L-side kernels for short tile columns: at most 32 rows a1 per tile and at
// most 32 key blocks c1, as with blocks of whole frames (b1 = f frames).
// k_aggregate and k_apply give one tile column (bh, g, a2) a workgroup of
// 128 rows and 64-key steps; a column of 21 rows and 21 keys would then use
// one wave of four and wait out a load latency for very little work.  Here
// each wave owns a column of its own, with its rows (and its keys and values)
// in 32-row LDS tiles of its own.  Per column the arithmetic is the other
// kernels', in the same order, so the results are the same.
#pragma once

#include "lside.h"

namespace monarch {

constexpr int kColsRows = 32;  // rows a1 per tile and key blocks c1 at most

// Global -> LDS DMA of a 32-row tile by the calling wave alone (TileDma
// splits a tile over the waves of a workgroup); same layout and row rule.
template <typename T, int D, int DK>
__device__ inline void wave_tile_dma(T* tile, const T* g, long long rstride, int nvalid) {
  constexpr int V = Elem<T>::kVec;
  constexpr int ROWB = DK * static_cast<int>(sizeof(T));
  constexpr int NINS = kColsRows * ROWB / 1024;
  static_assert(NINS * 1024 == kColsRows * ROWB, "tile must be a whole number of KiB");
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ci = 0; ci < NINS; ++ci) {
    const int byte = ci * 1024 + 16 * lane;
    const int r = byte / ROWB;
    const int c = ((byte % ROWB) / 16) ^ Tile<T, DK>::swz(r);  // logical chunk at this position
    int col = c * V;
    if (col >= D) col -= D;
    const int rr = r < nvalid ? r : nvalid - 1;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(g + rr * rstride + col),
                                     (__attribute__((address_space(3))) void*)(tile + ci * (1024 / static_cast<int>(sizeof(T)))),
                                     16, 0, 0);
  }
}

// Work item of a column kernel: NW consecutive columns of tile g; wave w
// takes column a2 = cg * NW + w (none when past b2).
struct ColsItem {
  int bh, g, a2, lo, nrows;
  bool valid;
  // work item wi of wn (default: this workgroup of the grid)
  __device__ ColsItem(const LGeom& p, int nw, int wave, int wi = -1, int wn = 0) {
    const int logical = wi < 0 ? xcd_remap(blockIdx.x, gridDim.x) : xcd_remap(wi, wn);
    const int ncg = (p.b2 + nw - 1) / nw;
    const int cg = logical % ncg;
    const int rest = logical / ncg;
    g = rest % p.t;
    bh = rest / p.t;
    a2 = cg * nw + wave;
    valid = a2 < p.b2;
    if (!valid) a2 = p.b2 - 1;  // keeps every address in range; nothing is stored
    lo = tile_lo(g, p.b1r, p.t);
    nrows = tile_lo(g + 1, p.b1r, p.t) - lo;
  }
};

// ---------------------------------------------------------- k_aggregate_cols --
// Qh[c1,:] = sum_(a1 in g) L[a1,c1] q_a1 / beta[c1] for one column per wave:
// the RW = 2 key tiles of the wave cover all b1 <= 32 keys, the column's rows
// form one 32-row block.
template <typename T, int D, int NW, bool BCAST>
__device__ __forceinline__ void k_aggregate_cols_item(const T* __restrict__ q, const T* __restrict__ kt,
                                                               const float* __restrict__ h2,
                                                               const float* __restrict__ lse,
                                                               T* __restrict__ qhat, float* __restrict__ beta_out,
                                                               LGeom p, const int* __restrict__ stop_at,
                                                               int it, int wi, int wn) {
  using E = Elem<T>;
  constexpr int RW = 2;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  __shared__ __align__(16) T sQ[NW][kColsRows * DK];
  __shared__ __align__(16) float sL[NW][64];

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const ColsItem ci(p, NW, wave, wi, wn);
  if (stop_at && stop_at[ci.bh] != 0 && stop_at[ci.bh] < it) return;  // head done iterating
  const int bh = ci.bh, g = ci.g, a2 = ci.a2, nrows = ci.nrows;
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);
  const T* qh = q + static_cast<long long>(bh) * p.N * D;
  const float* lh = lse + static_cast<long long>(bh) * p.N;
  const long long n_first = static_cast<long long>(ci.lo) * p.b2 + a2;
  wave_tile_dma<T, D, DK>(sQ[wave], qh + n_first * D, static_cast<long long>(p.b2) * D, nrows);
  dma_floats64(sL[wave], lh + n_first, p.b2, nrows);

  typename E::frag bk[RW][KS];
  float bias[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = rt * 16 + l16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bk[rt][s] = (c1 < p.b1 && col < D) ? E::load(ks.k + c1 * ks.kstride + col) : E::zero();
    }
    bias[rt] = BCAST ? 0.0f : (c1 < p.b1 ? ks.bias(c1, p.b1) : 0.0f);
  }
  f32x4 acc[NACC][2][RW];
  f32x4 accb[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    accb[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) acc[dp][0][rt] = acc[dp][1][rt] = f32x4{0, 0, 0, 0};
  }
  const typename E::frag ones = E::ones();
  __syncthreads();

  typename E::frag a[KS][2];
  typename E::frag v[NACC][2];
  load_rows<T, DK, KS>(a, sQ[wave], 0, l16, G);
  load_cols<T, D, DK, NACC>(v, sQ[wave], 0);
  float lr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lr[j] = sL[wave][8 * G + j];
  __builtin_amdgcn_sched_barrier(0);
  f32x4 S[2][RW];
  logits<T, KS, RW>(S, a, bk);
  typename E::frag pf[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, BCAST ? -lr[j] : bias[rt] - lr[j]));
      w[j] = 8 * G + j < nrows ? w[j] : 0.0f;
    }
    pf[rt] = E::pack(w);
    accb[rt] = E::mma(ones, pf[rt], accb[rt]);
  }
  weighted_sum<T, D, NACC, RW>(acc, v, pf);

  if (!ci.valid) return;
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const float b = accb[rt][0];
    const float inv = b > 0.0f ? 1.0f / b : 0.0f;
    const int c1 = rt * 16 + l16;
    if (c1 >= p.b1) continue;
    const long long row = ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2 + a2;
    store_rows<T, D, NACC, RW>(qhat + row * D, acc, rt, inv, G);
    if (beta_out && G == 0) beta_out[row] = b;
  }
}

// Work items k_aggregate_cols_item, one per workgroup, or looped over by fewer workgroups
// (nitems > 0); nothing runs once every head has stopped iterating (nstop).
template <typename T, int D, int NW, bool BCAST>
__global__ __launch_bounds__(NW * kWave) void k_aggregate_cols(const T* __restrict__ q, const T* __restrict__ kt,
                                                               const float* __restrict__ h2,
                                                               const float* __restrict__ lse,
                                                               T* __restrict__ qhat, float* __restrict__ beta_out,
                                                               LGeom p, const int* __restrict__ stop_at = nullptr,
                                                               int it = 0,
    const int* __restrict__ nstop = nullptr, int nitems = 0) {
  if (nstop && *nstop >= p.BH) return;
  const int wn = nitems > 0 ? nitems : static_cast<int>(gridDim.x);
  for (int wi = blockIdx.x; wi < wn; wi += gridDim.x) {
    if (wi != static_cast<int>(blockIdx.x)) __syncthreads();
    k_aggregate_cols_item<T, D, NW, BCAST>(q, kt, h2, lse, qhat, beta_out, p, stop_at, it, wi, wn);
  }
}

// ------------------------------------------------------------- k_apply_cols --
// y[a1,:] = sum_c1 L[a1,c1] U[g,c1,a2,:] for one column per wave: the column's
// rows are the wave's RW = 2 row tiles, its b1 <= 32 keys (and U rows) one
// 32-row LDS tile of its own (the block-mean keys are one tile shared by all).
template <typename T, int D, int NW, bool BCAST>
__global__ __launch_bounds__(NW * kWave) void k_apply_cols(const T* __restrict__ q, const T* __restrict__ kt,
                                                           const float* __restrict__ h2,
                                                           const float* __restrict__ lse, const T* __restrict__ u,
                                                           T* __restrict__ out, LGeom p) {
  using E = Elem<T>;
  constexpr int RW = 2;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  constexpr int NK = BCAST ? 1 : NW;  // key tiles
  __shared__ __align__(16) T sK[NK][kColsRows * DK];
  __shared__ __align__(16) T sU[NW][kColsRows * DK];
  __shared__ __align__(16) float sH[BCAST ? 1 : NW][BCAST ? 1 : 64];

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const ColsItem ci(p, NW, wave);
  const int bh = ci.bh, g = ci.g, a2 = ci.a2, nrows = ci.nrows;
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);
  const T* qh = q + static_cast<long long>(bh) * p.N * D;
  const float* lh = lse + static_cast<long long>(bh) * p.N;
  const T* ucol = u + ((static_cast<long long>(bh) * p.t + g) * p.b1 * p.b2 + a2) * D;
  const long long ustride = static_cast<long long>(p.b2) * D;
  if (BCAST) {
    TileDma<T, D, DK, kColsRows, NW>::issue(sK[0], ks.k, ks.kstride, p.b1);
  } else {
    wave_tile_dma<T, D, DK>(sK[BCAST ? 0 : wave], ks.k, ks.kstride, p.b1);
    dma_floats64(sH[BCAST ? 0 : wave], ks.h, ks.hstride, p.b1);
  }
  wave_tile_dma<T, D, DK>(sU[wave], ucol, ustride, p.b1);

  const long long n0 = static_cast<long long>(ci.lo) * p.b2 + a2;
  typename E::frag bq[RW][KS];
  float nlrow[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = rt * 16 + l16;
    const bool ok = r < nrows;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bq[rt][s] = (ok && col < D) ? E::load(qh + (n0 + static_cast<long long>(r) * p.b2) * D + col) : E::zero();
    }
    nlrow[rt] = ok ? -lh[n0 + static_cast<long long>(r) * p.b2] : 0.0f;
  }
  f32x4 acc[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) acc[dp][dt][rt] = f32x4{0, 0, 0, 0};
  __syncthreads();

  const T* cK = sK[BCAST ? 0 : wave];
  // keys past b1 only exist in this one block: weight 0
  const bool tail = kColsRows > p.b1;
  typename E::frag a[KS][2];
  typename E::frag v[NACC][2];
  load_rows<T, DK, KS>(a, cK, 0, l16, G);
  load_cols<T, D, DK, NACC>(v, sU[wave], 0);
  float bias[8];
  if (!BCAST) {
#pragma unroll
    for (int j = 0; j < 8; ++j) bias[j] = sH[BCAST ? 0 : wave][8 * G + j];
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 S[2][RW];
  logits<T, KS, RW>(S, a, bq);
  typename E::frag pf[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, BCAST ? nlrow[rt] : bias[j] + nlrow[rt]));
    if (tail) {
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = 8 * G + j < p.b1 ? w[j] : 0.0f;
    }
    pf[rt] = E::pack(w);
  }
  weighted_sum<T, D, NACC, RW>(acc, v, pf);

  if (!ci.valid) return;
  T* oh = out + static_cast<long long>(bh) * p.N * D;
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = rt * 16 + l16;
    if (r >= nrows) continue;
    store_rows<T, D, NACC, RW>(oh + (n0 + static_cast<long long>(r) * p.b2) * D, acc, rt, 1.0f, G);
  }
}

}  // namespace monarch
