// L-side kernels: everything indexed by a w-column a2 of the token grid.
//
// For one (batch*head, tile g, column a2) the L block is
//   L[a1, c1] = softmax_c1( s<q_(a1,a2), Kt[g,c1,a2]> + H[g,c1,a2] ),  a1 in tile g,
// (yunpan.plus MonarchRT article, section "Monarch matrices"; the L-step of
// MonarchAttention as read in the header of monarch_attn.h).  Query rows of
// the column are strided by b2*d in memory: that stride is the permutation
// P, applied as address arithmetic, never as a copy.
//
// Three passes share the same logits, computed with MFMA (bf16 in, fp32 out):
//   k_lse        log2-sum-exp of every L row (normaliser, needed by both others)
//   k_aggregate  Qh[g,c1,a2] = sum_a1 L q / sum_a1 L   (the R-step's "queries")
//   k_apply      y = L U with U[g,c1,a2] = R V         (the final product)
// Logits are in log2 units: x = c*<q,k> + h with c = log2(e)/sqrt(d), h = H*log2(e).
//
// Keys Kt come either from the block means of K (first iteration, R uniform:
// the same b1 x d matrix for every tile and column, BCAST) or from the
// previous R-step ([BH][t][b1][b2][d] with entropies h2 [BH][t][b1][b2]).
#pragma once

#include "device_common.h"

namespace monarch {

struct LGeom {
  int BH, N, b1, b2, t;
  int nrb;     // row blocks per (tile, column) or per head (contiguous mode)
  float c;     // log2(e) / sqrt(d)
};

// Keys (and entropy bias) of one (bh, g, a2) column.
template <typename T, int D, bool BCAST>
struct KeySrc {
  const T* k;
  long long kstride;   // elements between consecutive c1
  const float* h;
  int hstride;
  __device__ KeySrc(const T* kt, const float* h2, const LGeom& p, int bh, int g, int a2) {
    if (BCAST) {
      k = kt + static_cast<long long>(bh) * p.b1 * D;
      kstride = D;
      h = nullptr;
      hstride = 0;
    } else {
      const long long base = (static_cast<long long>(bh) * p.t + g) * p.b1 * p.b2 + a2;
      k = kt + base * D;
      kstride = static_cast<long long>(p.b2) * D;
      h = h2 + base;
      hstride = p.b2;
    }
  }
  __device__ float bias(int c1, int b1) const {
    if (c1 >= b1) return kNegInf;
    return BCAST ? 0.0f : h[static_cast<long long>(c1) * hstride] * kLog2e;
  }
};

// Work item of a per-column kernel: rows a1 in [a1_0, a1_0 + nrows) of tile g.
struct ColItem {
  int bh, g, a2, a1_0, nrows, lo, hi;
  __device__ ColItem(const LGeom& p, int rb_rows) {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int rb = logical % p.nrb;
    int rest = logical / p.nrb;
    a2 = rest % p.b2;
    rest /= p.b2;
    g = rest % p.t;
    bh = rest / p.t;
    lo = tile_lo(g, p.b1, p.t);
    hi = tile_lo(g + 1, p.b1, p.t);
    a1_0 = lo + rb * rb_rows;
    nrows = hi - a1_0 < rb_rows ? hi - a1_0 : rb_rows;
  }
};

// Fragment of the transposed tile for output columns of d-tile pair dp, half
// dt (pair mode: 8 consecutive d per lane after the product) or the single
// 16-wide d tile (D == 16).
template <typename T, int D>
__device__ inline typename Elem<T>::frag load_vals_tr(const T* tile, int pitch, int k0, int dp,
                                                      int dt) {
  if (D >= 32) return Elem<T>::load_tr(tile, pitch, k0, 32 * dp + 4 * dt, 8);
  return Elem<T>::load_tr(tile, pitch, k0, 0, 4);
}

// Store 8 (pair mode) or 4 (D == 16) consecutive outputs of lane group G.
template <typename T, int D, int NACC, int RW>
__device__ inline void store_rows(T* dst, const f32x4 (&acc)[NACC][2][RW], int rt, float scale,
                                  int G) {
  using E = Elem<T>;
  if (D >= 32) {
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = acc[dp][j >> 2][rt][j & 3] * scale;
      E::store8(dst + 32 * dp + 8 * G, v);
    }
  } else {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = acc[0][0][rt][i] * scale;
    E::store4(dst + 4 * G, v);
  }
}

// ------------------------------------------------------------------ k_lse --
// CONTIG: rows are consecutive tokens of a head (only with BCAST keys, where
// the logits do not depend on the column or tile).
template <typename T, int D, int RW, int NW, bool BCAST, bool CONTIG>
__global__ __launch_bounds__(NW * kWave) void k_lse(const T* __restrict__ q,
                                                    const T* __restrict__ kt,
                                                    const float* __restrict__ h2,
                                                    float* __restrict__ lse, LGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int PITCH = DK + E::kPad;
  constexpr int RB = NW * RW * 16;
  constexpr int NT = NW * kWave;
  __shared__ __align__(16) T sK[2][32 * PITCH];
  __shared__ float sBias[2][32];

  int bh, g = 0, a2 = 0, nrows;
  long long n0, nstride;
  if (CONTIG) {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    bh = logical / p.nrb;
    n0 = static_cast<long long>(logical % p.nrb) * RB;
    nstride = 1;
    nrows = p.N - n0 < RB ? static_cast<int>(p.N - n0) : RB;
  } else {
    ColItem it(p, RB);
    bh = it.bh; g = it.g; a2 = it.a2;
    n0 = static_cast<long long>(it.a1_0) * p.b2 + a2;
    nstride = p.b2;
    nrows = it.nrows;
  }
  if (nrows <= 0) return;
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const T* qh = q + static_cast<long long>(bh) * p.N * D;

  typename E::frag bq[RW][KS];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bq[rt][s] = (r < nrows && col < D) ? E::load(qh + (n0 + r * nstride) * D + col) : E::zero();
    }
  }

  float m[RW], l[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) { m[rt] = -1e30f; l[rt] = 0.0f; }

  TileLoader<T, D, DK, 32, NT> ld;
  const int nch = (p.b1 + 31) / 32;
  float bpre = 0.0f;
  ld.load(ks.k, ks.kstride, p.b1);
  if (threadIdx.x < 32) bpre = ks.bias(threadIdx.x, p.b1);
  ld.store(sK[0], PITCH);
  if (threadIdx.x < 32) sBias[0][threadIdx.x] = bpre;
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int cur = ch & 1;
    const bool more = ch + 1 < nch;
    if (more) {
      const int c1n = (ch + 1) * 32;
      ld.load(ks.k + c1n * ks.kstride, ks.kstride, p.b1 - c1n);
      if (threadIdx.x < 32) bpre = ks.bias(c1n + threadIdx.x, p.b1);
    }
    f32x4 S[2][RW];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) S[ct][rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const typename E::frag a = E::load(sK[cur] + perm_row(ct, l16) * PITCH + s * 32 + 8 * G);
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) S[ct][rt] = E::mma(a, bq[rt][s], S[ct][rt]);
      }
    }
    float bias[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bias[j] = sBias[cur][8 * G + j];
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      float x[8];
      float cm = -1e30f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = __builtin_fmaf(S[j >> 2][rt][j & 3], p.c, bias[j]);
        cm = fmaxf(cm, x[j]);
      }
      const float mn = fmaxf(m[rt], cm);
      float acc = l[rt] * fast_exp2(m[rt] - mn);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += fast_exp2(x[j] - mn);
      l[rt] = acc;
      m[rt] = mn;
    }
    if (more) {
      ld.store(sK[cur ^ 1], PITCH);
      if (threadIdx.x < 32) sBias[cur ^ 1][threadIdx.x] = bpre;
    }
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m[rt], off);
      const float lo = __shfl_xor(l[rt], off);
      const float mn = fmaxf(m[rt], mo);
      l[rt] = l[rt] * fast_exp2(m[rt] - mn) + lo * fast_exp2(mo - mn);
      m[rt] = mn;
    }
    const int r = (wave * RW + rt) * 16 + l16;
    if (G == 0 && r < nrows)
      lse[static_cast<long long>(bh) * p.N + n0 + r * nstride] = m[rt] + log2f(l[rt]);
  }
}

// ------------------------------------------------------------ k_aggregate --
// One workgroup: (bh, g, a2) and a block of CB = NW*RW*16 key blocks c1.
// Qh[c1,:] = sum_(a1 in g) L[a1,c1] q_a1 / sum_(a1 in g) L[a1,c1], computed as
// Qh^T = q^T P over chunks of 32 rows a1.  q is staged once, row-major: the
// logits read it by rows, the weighted sum reads it by columns (transposing
// LDS reads).
template <typename T, int D, int RW, int NW, bool BCAST>
__global__ __launch_bounds__(NW * kWave) void k_aggregate(const T* __restrict__ q,
                                                          const T* __restrict__ kt,
                                                          const float* __restrict__ h2,
                                                          const float* __restrict__ lse,
                                                          T* __restrict__ qhat, LGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int PITCH = DK + E::kPad;
  constexpr int CB = NW * RW * 16;
  constexpr int NT = NW * kWave;
  constexpr int NDP = D / 32;  // pairs of 16-wide d tiles (0 when D == 16)
  constexpr int NACC = NDP > 0 ? NDP : 1;
  __shared__ __align__(16) T sQ[2][32 * PITCH];
  __shared__ float sL[2][32];

  // decode (bh, g, a2, cb)
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nrb;
  int rest = logical / p.nrb;
  const int a2 = rest % p.b2;
  rest /= p.b2;
  const int g = rest % p.t;
  const int bh = rest / p.t;
  const int lo = tile_lo(g, p.b1, p.t), hi = tile_lo(g + 1, p.b1, p.t);
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;

  typename E::frag bk[RW][KS];
  float bias[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = cb * CB + (wave * RW + rt) * 16 + l16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bk[rt][s] = (c1 < p.b1 && col < D) ? E::load(ks.k + c1 * ks.kstride + col) : E::zero();
    }
    bias[rt] = ks.bias(c1, p.b1);
  }

  f32x4 acc[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) acc[dp][dt][rt] = f32x4{0, 0, 0, 0};
  float beta[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) beta[rt] = 0.0f;

  const T* qh = q + static_cast<long long>(bh) * p.N * D;
  const float* lh = lse + static_cast<long long>(bh) * p.N;
  const long long qstride = static_cast<long long>(p.b2) * D;
  const int nrows = hi - lo;
  const int nch = (nrows + 31) / 32;
  TileLoader<T, D, DK, 32, NT> ld;
  float lpre = 0.0f;
  auto fetch = [&](int ch) {
    const long long n_first = static_cast<long long>(lo + ch * 32) * p.b2 + a2;
    const int nvalid = nrows - ch * 32;
    ld.load(qh + n_first * D, qstride, nvalid);
    if (threadIdx.x < 32)
      lpre = static_cast<int>(threadIdx.x) < nvalid ? lh[n_first + threadIdx.x * static_cast<long long>(p.b2)]
                                                    : kPosInf;
  };
  fetch(0);
  ld.store(sQ[0], PITCH);
  if (threadIdx.x < 32) sL[0][threadIdx.x] = lpre;
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int cur = ch & 1;
    const bool more = ch + 1 < nch;
    if (more) fetch(ch + 1);

    f32x4 S[2][RW];
#pragma unroll
    for (int at = 0; at < 2; ++at)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) S[at][rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int at = 0; at < 2; ++at) {
        const typename E::frag a = E::load(sQ[cur] + perm_row(at, l16) * PITCH + s * 32 + 8 * G);
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) S[at][rt] = E::mma(a, bk[rt][s], S[at][rt]);
      }
    }
    float lrow[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) lrow[j] = sL[cur][8 * G + j];
    typename E::frag pf[RW];
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, bias[rt] - lrow[j]));
      pf[rt] = E::pack(w);
      float sb = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) sb += E::slot(pf[rt], j);
      beta[rt] += sb;
    }
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
      for (int dt = 0; dt < (NDP > 0 ? 2 : 1); ++dt) {
        const typename E::frag a = load_vals_tr<T, D>(sQ[cur], PITCH, 0, dp, dt);
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) acc[dp][dt][rt] = E::mma(a, pf[rt], acc[dp][dt][rt]);
      }
    if (more) {
      ld.store(sQ[cur ^ 1], PITCH);
      if (threadIdx.x < 32) sL[cur ^ 1][threadIdx.x] = lpre;
    }
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    float b = beta[rt];
    b += __shfl_xor(b, 16);
    b += __shfl_xor(b, 32);
    const float inv = b > 0.0f ? 1.0f / b : 0.0f;
    const int c1 = cb * CB + (wave * RW + rt) * 16 + l16;
    if (c1 >= p.b1) continue;
    T* dst = qhat + ((((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2 + a2) * D);
    store_rows<T, D, NACC, RW>(dst, acc, rt, inv, G);
  }
}

// ---------------------------------------------------------------- k_apply --
// One workgroup: (bh, g, a2) and a block of RB = NW*RW*16 rows a1 of tile g.
// y[a1,:] = sum_c1 L[a1,c1] U[g,c1,a2,:], with L normalised by the stored
// log-sum-exp (no running rescale), computed as y^T = U^T P^T.
template <typename T, int D, int RW, int NW, bool BCAST>
__global__ __launch_bounds__(NW * kWave) void k_apply(const T* __restrict__ q,
                                                      const T* __restrict__ kt,
                                                      const float* __restrict__ h2,
                                                      const float* __restrict__ lse,
                                                      const T* __restrict__ u,
                                                      T* __restrict__ out, LGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int PITCH = DK + E::kPad;
  constexpr int RB = NW * RW * 16;
  constexpr int NT = NW * kWave;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  __shared__ __align__(16) T sK[2][32 * PITCH];
  __shared__ __align__(16) T sU[2][32 * PITCH];
  __shared__ float sBias[2][32];

  ColItem it(p, RB);
  if (it.nrows <= 0) return;
  const int bh = it.bh, g = it.g, a2 = it.a2;
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);
  const long long n0 = static_cast<long long>(it.a1_0) * p.b2 + a2;
  const long long nstride = p.b2;

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const T* qh = q + static_cast<long long>(bh) * p.N * D;
  const float* lh = lse + static_cast<long long>(bh) * p.N;
  const T* ucol = u + ((static_cast<long long>(bh) * p.t + g) * p.b1 * p.b2 + a2) * D;
  const long long ustride = static_cast<long long>(p.b2) * D;

  typename E::frag bq[RW][KS];
  float lrow[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    const bool ok = r < it.nrows;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bq[rt][s] = (ok && col < D) ? E::load(qh + (n0 + r * nstride) * D + col) : E::zero();
    }
    lrow[rt] = ok ? lh[n0 + r * nstride] : 0.0f;
  }

  f32x4 acc[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) acc[dp][dt][rt] = f32x4{0, 0, 0, 0};

  TileLoader<T, D, DK, 32, NT> ldk;
  TileLoader<T, D, D, 32, NT> ldu;
  float bpre = 0.0f;
  const int nch = (p.b1 + 31) / 32;
  auto fetch = [&](int ch) {
    const int c1_0 = ch * 32;
    ldk.load(ks.k + c1_0 * ks.kstride, ks.kstride, p.b1 - c1_0);
    ldu.load(ucol + c1_0 * ustride, ustride, p.b1 - c1_0);
    if (threadIdx.x < 32) bpre = ks.bias(c1_0 + threadIdx.x, p.b1);
  };
  auto put = [&](int buf) {
    ldk.store(sK[buf], PITCH);
    ldu.store(sU[buf], PITCH);
    if (threadIdx.x < 32) sBias[buf][threadIdx.x] = bpre;
  };
  fetch(0);
  put(0);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int cur = ch & 1;
    const bool more = ch + 1 < nch;
    if (more) fetch(ch + 1);

    f32x4 S[2][RW];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) S[ct][rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const typename E::frag a = E::load(sK[cur] + perm_row(ct, l16) * PITCH + s * 32 + 8 * G);
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) S[ct][rt] = E::mma(a, bq[rt][s], S[ct][rt]);
      }
    }
    float bias[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bias[j] = sBias[cur][8 * G + j];
    typename E::frag pf[RW];
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, bias[j] - lrow[rt]));
      pf[rt] = E::pack(w);
    }
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
      for (int dt = 0; dt < (NDP > 0 ? 2 : 1); ++dt) {
        const typename E::frag a = load_vals_tr<T, D>(sU[cur], PITCH, 0, dp, dt);
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) acc[dp][dt][rt] = E::mma(a, pf[rt], acc[dp][dt][rt]);
      }
    if (more) put(cur ^ 1);
    __syncthreads();
  }

  T* oh = out + static_cast<long long>(bh) * p.N * D;
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    if (r >= it.nrows) continue;
    store_rows<T, D, NACC, RW>(oh + (n0 + r * nstride) * D, acc, rt, 1.0f, G);
  }
}

// ----------------------------------------------------------------- k_kbar --
// First L-step: with R uniform, every aggregated key is the block mean
// Kbar[c1] = (1/b2) sum_c2 k_(c1,c2), shared by all tiles and columns (and the
// entropy term log(b2) is the same for every c1, so it cancels in the softmax).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_kbar(const T* __restrict__ k, T* __restrict__ kbar,
                                              int BH, int b1, int b2) {
  using E = Elem<T>;
  constexpr int V = E::kVec;
  constexpr int LPR = D / V;        // lanes per row
  constexpr int RPI = kWave / LPR;  // rows per pass
  const long long item = static_cast<long long>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (item >= static_cast<long long>(BH) * b1) return;
  const int lane = lane_id();
  const int col = (lane % LPR) * V, ro = lane / LPR;
  const T* src = k + item * b2 * D;  // item = bh*b1 + c1 -> rows (bh*N + c1*b2 + c2)
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.0f;
  for (int c2 = ro; c2 < b2; c2 += RPI) {
    uint4 raw = *reinterpret_cast<const uint4*>(src + static_cast<long long>(c2) * D + col);
    const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] += E::to_f32(e[j]);
  }
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] += __shfl_xor(acc[j], off);
  if (ro == 0) {
    const float inv = 1.0f / static_cast<float>(b2);
    T* dst = kbar + item * D + col;
#pragma unroll
    for (int j = 0; j < V; ++j) dst[j] = E::from_f32(acc[j] * inv);
  }
}

}  // namespace monarch
