// Row-side backward kernels for short tile columns (at most 32 key blocks c1
// and at most 32 rows a1 per tile, as with blocks of whole frames): kb_du and
// kb_dq give a tile column a workgroup of 128 or 256 rows and 64-key steps;
// here, as in the forward's k_aggregate_cols / k_apply_cols, each wave owns a
// column of its own with its rows, keys and values in 32-row LDS tiles of its
// own.  Per element the arithmetic is kb_du's and kb_dq's, in the same order.
#pragma once

#include "backward.h"
#include "lside_cols.h"

namespace monarch {

// dU[g,c1,a2] = sum_(a1 in g) L[a1,c1] dy_(a1,a2) for one column per wave (the
// forward's aggregation with dy as the values, as kb_du).
template <typename T, int D, int NW, bool BCAST>
__global__ __launch_bounds__(NW * kWave) void kb_du_cols(const T* __restrict__ q, const T* __restrict__ dy,
                                                         const T* __restrict__ kt, const float* __restrict__ h2,
                                                         const float* __restrict__ lse, T* __restrict__ du,
                                                         LGeom p) {
  using E = Elem<T>;
  constexpr int RW = 2;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  __shared__ __align__(16) T sQ[NW][kColsRows * DK];
  __shared__ __align__(16) T sY[NW][kColsRows * DK];
  __shared__ __align__(16) float sL[NW][64];

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const ColsItem ci(p, NW, wave);
  const int bh = ci.bh, g = ci.g, a2 = ci.a2, nrows = ci.nrows;
  const long long n_first = static_cast<long long>(bh) * p.N + static_cast<long long>(ci.lo) * p.b2 + a2;
  const long long qstride = static_cast<long long>(p.b2) * D;
  wave_tile_dma<T, D, DK>(sQ[wave], q + n_first * D, qstride, nrows);
  wave_tile_dma<T, D, DK>(sY[wave], dy + n_first * D, qstride, nrows);
  dma_floats64(sL[wave], lse + n_first, p.b2, nrows);

  const long long gbase = (static_cast<long long>(bh) * p.t + g) * p.b1;  // (bh, g, c1 = 0)
  typename E::frag bk[RW][KS];
  float hb[RW];  // entropy bias of the lane's key block
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = rt * 16 + l16;
    const long long krow = BCAST ? static_cast<long long>(bh) * p.b1 + c1 : (gbase + c1) * p.b2 + a2;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bk[rt][s] = (c1 < p.b1 && col < D) ? E::load(kt + krow * D + col) : E::zero();
    }
    hb[rt] = (BCAST || c1 >= p.b1) ? 0.0f : h2[krow];
  }
  f32x4 acc[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) acc[dp][0][rt] = acc[dp][1][rt] = f32x4{0, 0, 0, 0};
  __syncthreads();

  typename E::frag a[KS][2];
  load_rows<T, DK, KS>(a, sQ[wave], 0, l16, G);
  float lr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lr[j] = sL[wave][8 * G + j];
  f32x4 S[2][RW];
  logits<T, KS, RW>(S, a, bk);
  typename E::frag pf[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, hb[rt] - lr[j]));
      w[j] = 8 * G + j < nrows ? w[j] : 0.0f;
    }
    pf[rt] = E::pack(w);
  }
  typename E::frag vv[NACC][2];
  load_cols<T, D, DK, NACC>(vv, sY[wave], 0);
  weighted_sum<T, D, NACC, RW>(acc, vv, pf);

  if (!ci.valid) return;
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = rt * 16 + l16;
    if (c1 >= p.b1) continue;
    store_rows<T, D, NACC, RW>(du + ((gbase + c1) * p.b2 + a2) * D, acc, rt, 1.0f, G);
  }
}

// kb_dq for one column per wave: pass 1 ghat = L G and eps = L e, delta =
// <dy,y> + <q,ghat> - eps; pass 2 dl = L (<dy,U> + <q,G> - e - delta),
// dq = ghat + s sum_c1 dl Kt and the stored s*dl.  All keys of the column
// are one 32-row block, so both passes share the staged tiles and the logits.
template <typename T, int D, int NW, bool BCAST, bool HAS_DY, int DQM>
__global__ __launch_bounds__(NW * kWave) void kb_dq_cols(const T* __restrict__ q, const T* __restrict__ dy,
                                                         const T* __restrict__ y, const T* __restrict__ kt,
                                                         const float* __restrict__ h2,
                                                         const float* __restrict__ lse, const T* __restrict__ u,
                                                         const T* __restrict__ gq, const float* __restrict__ ev,
                                                         T* __restrict__ dq, float* __restrict__ dq_acc,
                                                         T* __restrict__ dlout, int ldl, LGeom p, float sc) {
  using E = Elem<T>;
  constexpr int RW = 2;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  constexpr int TB = kColsRows * DK;
  __shared__ __align__(16) T sK[BCAST ? 1 : NW][TB];
  __shared__ __align__(16) T sU[HAS_DY ? NW : 1][HAS_DY ? TB : 8];
  __shared__ __align__(16) T sG[NW][TB];
  __shared__ __align__(16) float sE[NW][64];  // 64: one float per lane of the DMA
  __shared__ __align__(16) float sH[BCAST ? 1 : NW][BCAST ? 1 : 64];

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const ColsItem ci(p, NW, wave);
  const int bh = ci.bh, g = ci.g, a2 = ci.a2, nrows = ci.nrows;
  const long long hoff = static_cast<long long>(bh) * p.N;
  const long long n0 = static_cast<long long>(ci.lo) * p.b2 + a2;
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);
  const long long cbase = (static_cast<long long>(bh) * p.t + g) * p.b1 * p.b2 + a2;  // (bh, g, c1 = 0, a2)
  const long long ustride = static_cast<long long>(p.b2) * D;
  if (BCAST) {
    TileDma<T, D, DK, kColsRows, NW>::issue(sK[0], ks.k, ks.kstride, p.b1);
  } else {
    wave_tile_dma<T, D, DK>(sK[BCAST ? 0 : wave], ks.k, ks.kstride, p.b1);
    dma_floats64(sH[BCAST ? 0 : wave], ks.h, ks.hstride, p.b1);
  }
  wave_tile_dma<T, D, DK>(sG[wave], gq + cbase * D, ustride, p.b1);
  if (HAS_DY) wave_tile_dma<T, D, DK>(sU[HAS_DY ? wave : 0], u + cbase * D, ustride, p.b1);
  dma_floats64(sE[wave], ev + cbase, p.b2, p.b1);

  typename E::frag bq[RW][KS], bdy[RW][KS];
  float nl[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = rt * 16 + l16;
    const bool ok = r < nrows;
    const long long row = hoff + n0 + static_cast<long long>(r) * p.b2;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bq[rt][s] = (ok && col < D) ? E::load(q + row * D + col) : E::zero();
      bdy[rt][s] = (HAS_DY && ok && col < D) ? E::load(dy + row * D + col) : E::zero();
    }
    nl[rt] = ok ? -lse[row] : 0.0f;
  }
  f32x4 acc[NACC][2][RW];
  f32x4 acce[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    acce[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) acc[dp][0][rt] = acc[dp][1][rt] = f32x4{0, 0, 0, 0};
  }
  __syncthreads();

  const T* cK = sK[BCAST ? 0 : wave];
  const bool tail = kColsRows > p.b1;  // keys past b1: weight 0
  // ---------------- pass 1: ghat and eps
  typename E::frag a[KS][2];
  load_rows<T, DK, KS>(a, cK, 0, l16, G);
  f32x4 S[2][RW];
  logits<T, KS, RW>(S, a, bq);
  float e8[8], hb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    e8[j] = sE[wave][8 * G + j];
    hb[j] = BCAST ? 0.0f : sH[BCAST ? 0 : wave][8 * G + j];
  }
  {
    const typename E::frag ef = E::pack(e8);
    typename E::frag pf[RW];
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, nl[rt] + hb[j]));
      if (tail) {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = 8 * G + j < p.b1 ? w[j] : 0.0f;
      }
      pf[rt] = E::pack(w);
      acce[rt] = E::mma(ef, pf[rt], acce[rt]);
    }
    typename E::frag vv[NACC][2];
    load_cols<T, D, DK, NACC>(vv, sG[wave], 0);
    weighted_sum<T, D, NACC, RW>(acc, vv, pf);
  }

  // delta = <dy, y> + <q, ghat> - eps (every lane group holds a quarter of d)
  float dlt[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = rt * 16 + l16;
    const bool ok = r < nrows;
    const long long row = hoff + n0 + static_cast<long long>(ok ? r : 0) * p.b2;
    float part;
    if constexpr (D >= 32)
      part = dot_acc_frags<T, NACC, RW>(bq[rt], acc, rt);  // q of the row, held in bq
    else
      part = dot_acc_row<T, D, NACC, RW>(q + row * D, acc, rt, G);
    if (HAS_DY) {
      typename E::frag by[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int col = s * 32 + 8 * G;
        by[s] = (ok && col < D) ? E::load(y + row * D + col) : E::zero();
      }
      part += dot_frags<T, KS>(bdy[rt], by);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    dlt[rt] = part - acce[rt][0];
  }

  // ---------------- pass 2: dl and dq (the logits S of pass 1)
  {
    f32x4 X[2][RW];
    if (HAS_DY) {
      load_rows<T, DK, KS>(a, sU[HAS_DY ? wave : 0], 0, l16, G);
      logits<T, KS, RW>(X, a, bdy);  // <U, dy>
      load_rows<T, DK, KS>(a, sG[wave], 0, l16, G);
      products<T, KS, RW>(X, a, bq);  // + <G, q>
    } else {
      load_rows<T, DK, KS>(a, sG[wave], 0, l16, G);
      logits<T, KS, RW>(X, a, bq);  // <G, q>
    }
    typename E::frag pf[RW];
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w[j] = sc * fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, nl[rt] + hb[j])) *
               (X[j >> 2][rt][j & 3] - e8[j] - dlt[rt]);
      if (tail) {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = 8 * G + j < p.b1 ? w[j] : 0.0f;
      }
      pf[rt] = E::pack(w);
      // s*dl of row n, keys 8G .. 8G+7, for the key gradient
      const int r = rt * 16 + l16;
      if (ci.valid && r < nrows) {
        T* dst = dlout + (hoff + n0 + static_cast<long long>(r) * p.b2) * ldl + 8 * G;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint4*>(dst) = __builtin_bit_cast(uint4, pf[rt]);
        } else {
          E::store8(dst, w);
        }
      }
    }
    typename E::frag vv[NACC][2];
    load_cols<T, D, DK, NACC>(vv, cK, 0);
    weighted_sum<T, D, NACC, RW>(acc, vv, pf);
  }

  if (!ci.valid) return;
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = rt * 16 + l16;
    if (r >= nrows) continue;
    const long long row = hoff + n0 + static_cast<long long>(r) * p.b2;
    if (DQM == kDqAdd || DQM == kDqFinish) {
      // the lane's d positions, as store_rows lays them out
      const float* src = dq_acc + row * D;
#pragma unroll
      for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
        for (int dt = 0; dt < (D >= 32 ? 2 : 1); ++dt)
          acc[dp][dt][rt] += *reinterpret_cast<const f32x4*>(src + (D >= 32 ? 32 * dp + 8 * G + 4 * dt : 4 * G));
    }
    if (DQM == kDqInit || DQM == kDqAdd) {
      float* dst = dq_acc + row * D;
#pragma unroll
      for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
        for (int dt = 0; dt < (D >= 32 ? 2 : 1); ++dt)
          *reinterpret_cast<f32x4*>(dst + (D >= 32 ? 32 * dp + 8 * G + 4 * dt : 4 * G)) = acc[dp][dt][rt];
    } else {
      store_rows<T, D, NACC, RW>(dq + row * D, acc, rt, 1.0f, G);
    }
  }
}

}  // namespace monarch
