// Backward kernels of the one-iteration MonarchAttention: the gradient of
// sum(dy * y) with respect to q, k and v, as needed to finetune a video model
// with the attention in place (yunpan.plus MonarchRT article, "Innovation 3:
// finetuning and efficient kernels": the one-iteration form is trained).
//
// Forward with R starting uniform (keys of the L-step are the block means
// Kbar, whose entropy term is the same for every block and cancels):
//   L = softmax_c1(s<q_n, Kbar[c1]>), beta = sum_(a1 in g) L,
//   Qh = sum_(a1 in g) L q / beta, R = softmax_c2(s<Qh, k>), U = R V,
//   y_n = sum_c1 L U.
// Reverse (chain rule, in the order the kernels run):
//   kb_lcol<DU>     dU[g,c1,a2] = sum_(a1 in g) L dy
//   kb_rside        per key block c1: dR = <dU, v>, dz = R (dR - <R, dR>),
//                   G = s (sum_c2 dz k) / beta, e = <G, Qh>,
//                   dv = sum_(g,a2) R dU,  dk_R = s sum_(g,a2) dz Qh
//   kb_dq           per row n: ghat = sum_c1 L G, delta = <dy,y> + <q,ghat> - sum_c1 L e,
//                   dl = L (<dy,U> + <q,G> - e - delta), dq = ghat + s sum_c1 dl Kbar
//   kb_lcol<DKBAR>  dKbar[c1] = s sum_n dl q_n  (partial sums per tile and column group)
//   kb_dk_finish    dk = dk_R + dKbar / b2
// MFMA operand conventions and the slot permutation are those of the forward
// kernels (device_common.h); logits are in log2 units with c = log2(e)/sqrt(d)
// and the log-sum-exps saved by the forward are in the same units.
#pragma once

#include "lside.h"

namespace monarch {

struct BGeom {
  int BH, N, b1, b2, t;
  int ncb;     // key-block groups of a column pass
  int na2g;    // column groups per tile (column passes)
  int a2per;   // columns per group
  int b2p;     // b2 rounded up to 32 (key-block pass)
  float c;     // log2(e) / sqrt(d)
  float s;     // 1 / sqrt(d)
};

// S[ct][rt] += a[s][ct] * b[rt][s] over the contraction (no reset).
template <typename T, int KS, int RW>
__device__ inline void products(f32x4 (&S)[2][RW], const typename Elem<T>::frag (&a)[KS][2],
                                const typename Elem<T>::frag (&b)[RW][KS]) {
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) S[ct][rt] = Elem<T>::mma(a[s][ct], b[rt][s], S[ct][rt]);
}

// Sum over the lane's d positions of x[d] * acc[d], where acc is an output
// tile of a weighted sum (lane holds d = 32dp + 8G + j, or 4G + i when
// D == 16) and x is read from row `xrow` of global memory (or NULL: 0).
template <typename T, int D, int NACC, int RW>
__device__ inline float dot_acc_row(const T* xrow, const f32x4 (&acc)[NACC][2][RW], int rt, int G) {
  float r = 0.0f;
  if (D >= 32) {
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) {
      const typename Elem<T>::frag x = Elem<T>::load(xrow + 32 * dp + 8 * G);
#pragma unroll
      for (int j = 0; j < 8; ++j) r += Elem<T>::slot(x, j) * acc[dp][j >> 2][rt][j & 3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r += Elem<T>::to_f32(xrow[4 * G + i]) * acc[0][0][rt][i];
  }
  return r;
}

// Sum over the lane's contraction slots of two row fragments (same layout).
template <typename T, int KS>
__device__ inline float dot_frags(const typename Elem<T>::frag (&a)[KS], const typename Elem<T>::frag (&b)[KS]) {
  float r = 0.0f;
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) r += Elem<T>::slot(a[s], j) * Elem<T>::slot(b[s], j);
  return r;
}

// --------------------------------------------------------------- kb_lcol --
// Column pass: one workgroup owns CB = NW*RW*16 key blocks c1 of tile g and a
// group of columns a2; the rows a1 of the tile stream through LDS in steps of
// 64, column after column, double-buffered by DMA.
//   DU:    dU[g,c1,a2] = sum_(a1 in g) L[a1,c1] dy_(a1,a2)      (groups of one column)
//   DKBAR: part[g*na2g + group][c1] = s sum_(a2 in group) sum_(a1 in g) dl q
enum { kLcolDU = 0, kLcolDKbar = 1 };

template <typename T, int D, int RW, int NW, int MODE>
__global__ __launch_bounds__(NW * kWave) void kb_lcol(const T* __restrict__ q, const T* __restrict__ dy,
                                                      const T* __restrict__ kbar, const float* __restrict__ lse,
                                                      const float* __restrict__ delta, const T* __restrict__ u,
                                                      const T* __restrict__ gq, const float* __restrict__ ev,
                                                      T* __restrict__ du, float* __restrict__ part, BGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int CB = NW * RW * 16;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  constexpr bool DKB = MODE == kLcolDKbar;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  __shared__ __align__(16) T sQ[2][kStep * DK];
  __shared__ __align__(16) T sY[2][kStep * DK];
  __shared__ __align__(16) float sLs[2][kStep];
  __shared__ __align__(16) float sDl[2][kStep];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.ncb;
  int rest = logical / p.ncb;
  const int a2g = rest % p.na2g;
  rest /= p.na2g;
  const int g = rest % p.t;
  const int bh = rest / p.t;
  const int lo = tile_lo(g, p.b1, p.t), hi = tile_lo(g + 1, p.b1, p.t);
  const int nrows = hi - lo;
  const int a2_0 = a2g * p.a2per;
  const int ncol = p.b2 - a2_0 < p.a2per ? p.b2 - a2_0 : p.a2per;
  if (ncol <= 0 || nrows <= 0) return;  // uniform over the workgroup
  const int nsteps = (nrows + kStep - 1) / kStep;
  const int nst = ncol * nsteps;

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const long long hoff = static_cast<long long>(bh) * p.N;
  const T* qh = q + hoff * D;
  const T* dyh = dy + hoff * D;
  const long long qstride = static_cast<long long>(p.b2) * D;
  const long long gbase = (static_cast<long long>(bh) * p.t + g) * p.b1;  // (bh, g, c1 = 0)

  auto fetch = [&](int st, int buf) {
    const int col = a2_0 + st / nsteps, step = st % nsteps;
    const long long n_first = static_cast<long long>(lo + step * kStep) * p.b2 + col;
    const int nvalid = nrows - step * kStep;
    Dma::issue(sQ[buf], qh + n_first * D, qstride, nvalid);
    Dma::issue(sY[buf], dyh + n_first * D, qstride, nvalid);
    if (wave == NW - 1) dma_floats64(sLs[buf], lse + hoff + n_first, p.b2, nvalid);
    if (DKB && wave == 0) dma_floats64(sDl[buf], delta + hoff + n_first, p.b2, nvalid);
  };
  fetch(0, 0);

  // the wave's key blocks as B operands; U, G, e of the current column
  typename E::frag bk[RW][KS], bu[RW][KS], bg[RW][KS];
  float ee[RW];
  int c1v[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = cb * CB + (wave * RW + rt) * 16 + l16;
    c1v[rt] = c1;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bk[rt][s] = (c1 < p.b1 && col < D) ? E::load(kbar + (static_cast<long long>(bh) * p.b1 + c1) * D + col)
                                         : E::zero();
    }
  }
  auto load_col = [&](int a2) {
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      const bool ok = c1v[rt] < p.b1;
      const long long row = (gbase + (ok ? c1v[rt] : 0)) * p.b2 + a2;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int col = s * 32 + 8 * G;
        bu[rt][s] = (ok && col < D) ? E::load(u + row * D + col) : E::zero();
        bg[rt][s] = (ok && col < D) ? E::load(gq + row * D + col) : E::zero();
      }
      ee[rt] = ok ? ev[row] : 0.0f;
    }
  };
  if (DKB) load_col(a2_0);

  f32x4 acc[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) acc[dp][dt][rt] = f32x4{0, 0, 0, 0};
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    const int step = st % nsteps;
    if (st + 1 < nst) fetch(st + 1, cur ^ 1);
    if (DKB && step == 0 && st > 0) load_col(a2_0 + st / nsteps);
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
      const int k0 = 32 * half;
      const int r0 = step * kStep + k0;
      if (r0 >= nrows) break;
      const bool tail = r0 + 32 > nrows;
      typename E::frag a[KS][2];
      load_rows<T, DK, KS>(a, sQ[cur], k0, l16, G);
      float lr[8], dl8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lr[j] = sLs[cur][k0 + 8 * G + j];
        dl8[j] = DKB ? sDl[cur][k0 + 8 * G + j] : 0.0f;
      }
      f32x4 S[2][RW], X[2][RW];
      logits<T, KS, RW>(S, a, bk);
      if (DKB) {
        logits<T, KS, RW>(X, a, bg);  // <q, G>
        typename E::frag ay[KS][2];
        load_rows<T, DK, KS>(ay, sY[cur], k0, l16, G);
        products<T, KS, RW>(X, ay, bu);  // + <dy, U>
      }
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, -lr[j]));
          if (DKB) w[j] *= X[j >> 2][rt][j & 3] - ee[rt] - dl8[j];
        }
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = r0 + 8 * G + j < nrows ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, DKB ? sQ[cur] : sY[cur], k0);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = c1v[rt];
    if (c1 >= p.b1) continue;
    if (DKB) {
      float* dst = part + ((static_cast<long long>(bh) * p.t * p.na2g + g * p.na2g + a2g) * p.b1 + c1) * D;
      store_rows<float, D, NACC, RW>(dst, acc, rt, p.s, G);
    } else {
      store_rows<T, D, NACC, RW>(du + ((gbase + c1) * p.b2 + a2_0) * D, acc, rt, 1.0f, G);
    }
  }
}

// --------------------------------------------------------------- kb_rside --
// Key-block pass: one workgroup per (bh, c1) with ceil(b2/16) waves, looping
// over the tiles g.  K and V of the block stay in LDS; per tile the
// aggregated queries Qh and dU (b2 x d each, contiguous) are copied in.
//   phase A, wave = 16 rows a2: R (logits transposed, softmax over c2), dR,
//     rho = <R, dR>, dz, dQh = s K^T dz -> G = dQh / beta, e = <G, Qh>;
//     the row statistics go to LDS for phase B.
//   phase B, wave = 16 keys c2: R and dz again with a2 as the contraction
//     (operands swap roles), dv^T += dU^T R and dk_R^T += Qh^T dz.
template <typename T, int D>
inline size_t rside_bwd_lds_bytes(int b2p) {
  const int DK = D < 32 ? 32 : D;
  return sizeof(T) * static_cast<size_t>(b2p) * DK * 4 + sizeof(float) * 2 * b2p;
}

// Global -> LDS DMA of `rows` rows of a contiguous [rows][D] block into a
// swizzled tile (rows >= nvalid repeat row nvalid-1).
template <typename T, int D, int DK>
__device__ inline void dma_block(T* tile, const T* src, int rows, int nvalid, int nw) {
  constexpr int V = Elem<T>::kVec;
  constexpr int ROWB = DK * static_cast<int>(sizeof(T));
  const int nins = rows * ROWB / 1024;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  for (int ci = wave; ci < nins; ci += nw) {
    const int byte = ci * 1024 + 16 * lane;
    const int r = byte / ROWB;
    const int c = ((byte % ROWB) / 16) ^ Tile<T, DK>::swz(r);
    int col = c * V;
    if (col >= D) col -= D;
    const long long off = static_cast<long long>(r < nvalid ? r : nvalid - 1) * D + col;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + off),
                                     (__attribute__((address_space(3))) void*)(tile + ci * (1024 / static_cast<int>(sizeof(T)))),
                                     16, 0, 0);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(512) void kb_rside(const T* __restrict__ k, const T* __restrict__ v,
                                                const T* __restrict__ qhat, const T* __restrict__ du,
                                                const float* __restrict__ beta, T* __restrict__ gq,
                                                float* __restrict__ ev, T* __restrict__ dv,
                                                float* __restrict__ dkr, BGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  using TL = Tile<T, DK>;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  constexpr int MAXCP = 4;  // b2 <= 128
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int b2p = p.b2p;
  T* sK = reinterpret_cast<T*>(smem_raw);
  T* sV = sK + b2p * DK;
  T* sQh = sV + b2p * DK;
  T* sDU = sQh + b2p * DK;
  float* sLR = reinterpret_cast<float*>(sDU + b2p * DK);
  float* sRho = sLR + b2p;

  const int item = xcd_remap(blockIdx.x, gridDim.x);  // bh*b1 + c1
  const int c1 = item % p.b1;
  const int bh = item / p.b1;
  const long long blk = static_cast<long long>(item) * p.b2;  // first key row of block c1
  const int nw = blockDim.x / kWave;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const int ncp = b2p / 32;
  const int mine = wave * 16 + l16;  // a2 in phase A, c2 in phase B

  dma_block<T, D, DK>(sK, k + blk * D, b2p, p.b2, nw);
  dma_block<T, D, DK>(sV, v + blk * D, b2p, p.b2, nw);
  f32x4 accv[NACC][2][1], acck[NACC][2][1];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      accv[dp][dt][0] = f32x4{0, 0, 0, 0};
      acck[dp][dt][0] = f32x4{0, 0, 0, 0};
    }

  for (int g = 0; g < p.t; ++g) {
    const long long rb = ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2;  // row (g, c1, a2 = 0)
    dma_block<T, D, DK>(sQh, qhat + rb * D, b2p, p.b2, nw);
    dma_block<T, D, DK>(sDU, du + rb * D, b2p, p.b2, nw);
    __syncthreads();

    // ---------------- phase A: columns a2 = mine of the transposed tiles
    {
      typename E::frag bq[KS], bd[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int col = 32 * s + 8 * G;
        bq[s] = col < D ? TL::load8(sQh, mine, col) : E::zero();
        bd[s] = col < D ? TL::load8(sDU, mine, col) : E::zero();
      }
      f32x4 S[MAXCP][2], DR[MAXCP][2];
#pragma unroll
      for (int cp = 0; cp < MAXCP; ++cp) {
        S[cp][0] = S[cp][1] = DR[cp][0] = DR[cp][1] = f32x4{0, 0, 0, 0};
        if (cp < ncp) {
#pragma unroll
          for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              const int r = 32 * cp + perm_row(ct, l16);
              S[cp][ct] = E::mma(TL::load8(sK, r, 32 * s + 8 * G), bq[s], S[cp][ct]);
              DR[cp][ct] = E::mma(TL::load8(sV, r, 32 * s + 8 * G), bd[s], DR[cp][ct]);
            }
        }
      }
      // softmax over c2 = 32cp + 8G + j (lane column a2)
      float x[MAXCP][8];
      float mx = -1e30f;
#pragma unroll
      for (int cp = 0; cp < MAXCP; ++cp)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c2 = 32 * cp + 8 * G + j;
          x[cp][j] = (cp < ncp && c2 < p.b2) ? S[cp][j >> 2][j & 3] * p.c : kNegInf;
          mx = fmaxf(mx, x[cp][j]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float sum = 0.0f;
#pragma unroll
      for (int cp = 0; cp < MAXCP; ++cp)
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += fast_exp2(x[cp][j] - mx);
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const float lse2 = mx + log2f(sum);
      float rho = 0.0f;
#pragma unroll
      for (int cp = 0; cp < MAXCP; ++cp)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x[cp][j] = fast_exp2(x[cp][j] - lse2);  // now R
          rho += x[cp][j] * DR[cp][j >> 2][j & 3];
        }
      rho += __shfl_xor(rho, 16);
      rho += __shfl_xor(rho, 32);
      // dQh^T = K^T dz^T: rows d, columns a2
      f32x4 acc[NACC][2][1];
#pragma unroll
      for (int dp = 0; dp < NACC; ++dp) acc[dp][0][0] = acc[dp][1][0] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int cp = 0; cp < MAXCP; ++cp) {
        if (cp >= ncp) break;
        float z[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = x[cp][j] * (DR[cp][j >> 2][j & 3] - rho);
        const typename E::frag zf = E::pack(z);
#pragma unroll
        for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
          for (int dt = 0; dt < (NDP > 0 ? 2 : 1); ++dt)
            acc[dp][dt][0] = E::mma(load_vals_tr<T, D, DK>(sK, 32 * cp, dp, dt), zf, acc[dp][dt][0]);
      }
      if (G == 0 && mine < b2p) {
        sLR[mine] = lse2;
        sRho[mine] = rho;
      }
      const bool ok = mine < p.b2;
      const float bt = ok ? beta[rb + mine] : 0.0f;
      const float sc = bt > 0.0f ? p.s / bt : 0.0f;
#pragma unroll
      for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) acc[dp][dt][0] *= sc;
      // e = <G, Qh> with the rounded Qh the forward used
      float e = 0.0f;
      if (D >= 32) {
#pragma unroll
        for (int dp = 0; dp < NACC; ++dp) {
          const typename E::frag xq = TL::load8(sQh, mine, 32 * dp + 8 * G);
#pragma unroll
          for (int j = 0; j < 8; ++j) e += E::slot(xq, j) * acc[dp][j >> 2][0][j & 3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) e += E::to_f32(sQh[TL::off(mine, 4 * G + i)]) * acc[0][0][0][i];
      }
      e += __shfl_xor(e, 16);
      e += __shfl_xor(e, 32);
      if (ok) {
        store_rows<T, D, NACC, 1>(gq + (rb + mine) * D, acc, 0, 1.0f, G);
        if (G == 0) ev[rb + mine] = e;
      }
    }
    __syncthreads();

    // ---------------- phase B: keys c2 = mine, contraction over a2
    // the wave's keys and values by rows as B operands (columns >= D zero)
    typename E::frag bk2[1][KS], bv2[1][KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = 32 * s + 8 * G;
      bk2[0][s] = col < D ? TL::load8(sK, mine, col) : E::zero();
      bv2[0][s] = col < D ? TL::load8(sV, mine, col) : E::zero();
    }
#pragma unroll 1
    for (int k0 = 0; k0 < b2p; k0 += 32) {
      typename E::frag a[KS][2];
      f32x4 Z[2][1], DR[2][1];
      load_rows<T, DK, KS>(a, sQh, k0, l16, G);
      logits<T, KS, 1>(Z, a, bk2);
      load_rows<T, DK, KS>(a, sDU, k0, l16, G);
      logits<T, KS, 1>(DR, a, bv2);
      float r[8], z[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int a2 = k0 + 8 * G + j;
        // rows a2 >= b2 are padding (their statistics were never written)
        r[j] = a2 < p.b2 ? fast_exp2(Z[j >> 2][0][j & 3] * p.c - sLR[a2]) : 0.0f;
        z[j] = a2 < p.b2 ? r[j] * (DR[j >> 2][0][j & 3] - sRho[a2]) : 0.0f;
      }
      typename E::frag rf[1] = {E::pack(r)}, zf[1] = {E::pack(z)};
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, sDU, k0);
      weighted_sum<T, D, NACC, 1>(accv, vv, rf);
      load_cols<T, D, DK, NACC>(vv, sQh, k0);
      weighted_sum<T, D, NACC, 1>(acck, vv, zf);
    }
    __syncthreads();
  }

  if (mine < p.b2) {
    store_rows<T, D, NACC, 1>(dv + (blk + mine) * D, accv, 0, 1.0f, G);
    store_rows<float, D, NACC, 1>(dkr + (blk + mine) * D, acck, 0, p.s, G);
  }
}

// ------------------------------------------------------------------ kb_dq --
// Row pass (as k_apply): one workgroup owns RB = NW*RW*16 rows a1 of tile g
// in column a2.  Pass 1 over c1: ghat = sum L G and eps = sum L e (a product
// with e in every row of the A operand), then delta = <dy,y> + <q,ghat> - eps
// (written out for the key-mean pass).  Pass 2 over c1:
// dl = L (<dy,U> + <q,G> - e - delta) and dq = ghat + s sum_c1 dl Kbar.
template <typename T, int D, int RW, int NW>
__global__ __launch_bounds__(NW * kWave) void kb_dq(const T* __restrict__ q, const T* __restrict__ dy,
                                                    const T* __restrict__ y, const T* __restrict__ kbar,
                                                    const float* __restrict__ lse, const T* __restrict__ u,
                                                    const T* __restrict__ gq, const float* __restrict__ ev,
                                                    float* __restrict__ delta, T* __restrict__ dq, LGeom p,
                                                    float sc) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int RB = NW * RW * 16;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  // double-buffered for bf16; f32 tiles are twice as large: one buffer
  constexpr int NB = sizeof(T) == 2 ? 2 : 1;
  __shared__ __align__(16) T sK[NB][kStep * DK];
  __shared__ __align__(16) T sU[NB][kStep * DK];
  __shared__ __align__(16) T sG[NB][kStep * DK];
  __shared__ __align__(16) float sE[NB][kStep];

  ColItem it(p, RB);
  if (it.nrows <= 0) return;
  const int bh = it.bh, g = it.g, a2 = it.a2;
  const long long hoff = static_cast<long long>(bh) * p.N;
  const long long n0 = static_cast<long long>(it.a1_0) * p.b2 + a2;
  const long long nstride = p.b2;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const T* kb = kbar + static_cast<long long>(bh) * p.b1 * D;
  const long long cbase = (static_cast<long long>(bh) * p.t + g) * p.b1 * p.b2 + a2;  // (bh, g, c1 = 0, a2)
  const long long ustride = static_cast<long long>(p.b2) * D;

  const int nst = (p.b1 + kStep - 1) / kStep;
  auto fetch = [&](int st, int buf, bool with_u) {
    const int c1 = st * kStep;
    Dma::issue(sK[buf], kb + static_cast<long long>(c1) * D, D, p.b1 - c1);
    Dma::issue(sG[buf], gq + (cbase + static_cast<long long>(c1) * p.b2) * D, ustride, p.b1 - c1);
    if (with_u) Dma::issue(sU[buf], u + (cbase + static_cast<long long>(c1) * p.b2) * D, ustride, p.b1 - c1);
    if (wave == NW - 1) dma_floats64(sE[buf], ev + cbase + static_cast<long long>(c1) * p.b2, p.b2, p.b1 - c1);
  };
  fetch(0, 0, false);

  typename E::frag bq[RW][KS], bdy[RW][KS];
  float nl[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    const bool ok = r < it.nrows;
    const long long row = hoff + n0 + r * nstride;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bq[rt][s] = (ok && col < D) ? E::load(q + row * D + col) : E::zero();
      bdy[rt][s] = (ok && col < D) ? E::load(dy + row * D + col) : E::zero();
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

  // ---------------- pass 1: ghat and eps
  for (int st = 0; st < nst; ++st) {
    const int cur = st % NB;
    if (NB == 2 && st + 1 < nst) fetch(st + 1, cur ^ 1, false);
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
      const int k0 = 32 * half;
      const int c1_0 = st * kStep + k0;
      if (c1_0 >= p.b1) break;
      const bool tail = c1_0 + 32 > p.b1;
      typename E::frag a[KS][2];
      load_rows<T, DK, KS>(a, sK[cur], k0, l16, G);
      f32x4 S[2][RW];
      logits<T, KS, RW>(S, a, bq);
      float e8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e8[j] = sE[cur][k0 + 8 * G + j];
      const typename E::frag ef = E::pack(e8);
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, nl[rt]));
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = c1_0 + 8 * G + j < p.b1 ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
        acce[rt] = E::mma(ef, pf[rt], acce[rt]);
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, sG[cur], k0);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    __syncthreads();
    if (NB == 1 && st + 1 < nst) {
      fetch(st + 1, 0, false);
      __syncthreads();
    }
  }
  fetch(0, 0, true);

  // delta = <dy, y> + <q, ghat> - eps (every lane group holds a quarter of d)
  float dlt[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    const bool ok = r < it.nrows;
    const long long row = hoff + n0 + (ok ? r : 0) * nstride;
    typename E::frag by[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      by[s] = (ok && col < D) ? E::load(y + row * D + col) : E::zero();
    }
    float part = dot_frags<T, KS>(bdy[rt], by) + dot_acc_row<T, D, NACC, RW>(q + row * D, acc, rt, G);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    dlt[rt] = part - acce[rt][0];
    if (ok && G == 0) delta[row] = dlt[rt];
  }
  __syncthreads();

  // ---------------- pass 2: dl and dq
  for (int st = 0; st < nst; ++st) {
    const int cur = st % NB;
    if (NB == 2 && st + 1 < nst) fetch(st + 1, cur ^ 1, true);
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
      const int k0 = 32 * half;
      const int c1_0 = st * kStep + k0;
      if (c1_0 >= p.b1) break;
      const bool tail = c1_0 + 32 > p.b1;
      typename E::frag a[KS][2];
      f32x4 S[2][RW], X[2][RW];
      load_rows<T, DK, KS>(a, sK[cur], k0, l16, G);
      logits<T, KS, RW>(S, a, bq);
      load_rows<T, DK, KS>(a, sU[cur], k0, l16, G);
      logits<T, KS, RW>(X, a, bdy);  // <U, dy>
      load_rows<T, DK, KS>(a, sG[cur], k0, l16, G);
      products<T, KS, RW>(X, a, bq);  // + <G, q>
      float e8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e8[j] = sE[cur][k0 + 8 * G + j];
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[j] = sc * fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, nl[rt])) *
                 (X[j >> 2][rt][j & 3] - e8[j] - dlt[rt]);
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = c1_0 + 8 * G + j < p.b1 ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, sK[cur], k0);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    __syncthreads();
    if (NB == 1 && st + 1 < nst) {
      fetch(st + 1, 0, true);
      __syncthreads();
    }
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    if (r >= it.nrows) continue;
    store_rows<T, D, NACC, RW>(dq + (hoff + n0 + r * nstride) * D, acc, rt, 1.0f, G);
  }
}

// ----------------------------------------------------------- kb_dk_finish --
// dk[c1,c2,:] = dk_R[c1,c2,:] + (sum of the key-mean partials)[c1,:] / b2.
// One thread per (bh, c1, 4 consecutive d), looping over c2.
template <typename T, int D>
__global__ __launch_bounds__(256) void kb_dk_finish(const float* __restrict__ dkr, const float* __restrict__ part,
                                                    T* __restrict__ dk, int BH, int b1, int b2, int np) {
  using E = Elem<T>;
  constexpr int CH = D / 4;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long long>(BH) * b1 * CH) return;
  const int ch = static_cast<int>(idx % CH);
  const long long bc = idx / CH;  // bh*b1 + c1
  const int bh = static_cast<int>(bc / b1), c1 = static_cast<int>(bc % b1);
  f32x4 m = f32x4{0, 0, 0, 0};
  for (int i = 0; i < np; ++i)
    m += *reinterpret_cast<const f32x4*>(part + ((static_cast<long long>(bh) * np + i) * b1 + c1) * D + 4 * ch);
  m *= 1.0f / static_cast<float>(b2);
  for (int c2 = 0; c2 < b2; ++c2) {
    const long long off = (bc * b2 + c2) * D + 4 * ch;
    const f32x4 r = *reinterpret_cast<const f32x4*>(dkr + off) + m;
    const float o[4] = {r[0], r[1], r[2], r[3]};
    E::store4(dk + off, o);
  }
}

}  // namespace monarch
