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

#include <type_traits>

#include "device_common.h"

namespace monarch {

struct LGeom {
  int BH;
  int N;       // query tokens per head (rows of q, lse, out)
  int b1;      // key blocks c1
  int b1r;     // query blocks a1 (== b1 for the square layer; fewer for a chunk of frames)
  int b2, t;
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
  // entropy bias of key block c1 in log2 units (the R-step stores it in bits)
  __device__ float bias(int c1, int b1) const {
    if (c1 >= b1) return kNegInf;
    return BCAST ? 0.0f : h[static_cast<long long>(c1) * hstride];
  }
};

// Work item of a per-column kernel: rows a1 in [a1_0, a1_0 + nrows) of tile g.
struct ColItem {
  int bh, g, a2, a1_0, nrows, lo, hi;
  // work item wi of wn (default: this workgroup of the grid)
  __device__ ColItem(const LGeom& p, int rb_rows, int wi = -1, int wn = 0) {
    const int logical = wi < 0 ? xcd_remap(blockIdx.x, gridDim.x) : xcd_remap(wi, wn);
    const int rb = logical % p.nrb;
    int rest = logical / p.nrb;
    a2 = rest % p.b2;
    rest /= p.b2;
    g = rest % p.t;
    bh = rest / p.t;
    lo = tile_lo(g, p.b1r, p.t);
    hi = tile_lo(g + 1, p.b1r, p.t);
    a1_0 = lo + rb * rb_rows;
    nrows = hi - a1_0 < rb_rows ? hi - a1_0 : rb_rows;
  }
};

// Rows of K, q or U staged per pipeline step (32-row MFMA contraction
// blocks); one barrier per step.
#ifndef MONARCH_STEP
#define MONARCH_STEP 64
#endif
constexpr int kStep = MONARCH_STEP;
constexpr int kHalves = kStep / 32;
static_assert(kStep == 64, "one 64-lane float DMA stages the log-sum-exps / entropies of a step");
// Minimum waves per SIMD the register allocator must allow (launch bounds).
#ifndef MONARCH_LSE_MINW
#define MONARCH_LSE_MINW 4
#endif
// the first L-step's form (keys shared by all columns)
#ifndef MONARCH_LSE_MINW_BCAST
#define MONARCH_LSE_MINW_BCAST 4
#endif
#ifndef MONARCH_AGG_MINW
#define MONARCH_AGG_MINW 1
#endif
#ifndef MONARCH_APP_MINW
#define MONARCH_APP_MINW 1
#endif
#ifndef MONARCH_ROWSKIP
#define MONARCH_ROWSKIP 1
#endif
#ifndef MONARCH_AGG_HALF
#define MONARCH_AGG_HALF 1
#endif

// Fragment of a transposed tile for output columns of d-tile pair dp, half dt
// (pair mode: the product leaves 8 consecutive d per lane) or the single
// 16-wide d tile (D == 16), contraction rows k0..k0+31.
template <typename T, int D, int DK>
__device__ inline typename Elem<T>::frag load_vals_tr(const T* tile, int k0, int dp, int dt) {
  if (D >= 32) return Tile<T, DK>::load_tr(tile, k0, 32 * dp + 4 * dt, 8);
  return Tile<T, DK>::load_tr(tile, k0, 0, 4);
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

// The 32-row block k0..k0+31 of a tile as A fragments by rows (permuted, see
// perm_row), for logits: a[s][ct] covers contraction columns 32s..32s+31.
template <typename T, int DK, int KS>
__device__ inline void load_rows(typename Elem<T>::frag (&a)[KS][2], const T* tile, int k0, int l16,
                                 int G) {
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) a[s][ct] = Tile<T, DK>::load8(tile, k0 + perm_row(ct, l16), s * 32 + 8 * G);
}

// The same block by columns, for the weighted sums: v[dp][dt] (see load_vals_tr).
template <typename T, int D, int DK, int NACC>
__device__ inline void load_cols(typename Elem<T>::frag (&v)[NACC][2], const T* tile, int k0) {
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < (D >= 32 ? 2 : 1); ++dt) v[dp][dt] = load_vals_tr<T, D, DK>(tile, k0, dp, dt);
}

// S tiles with rows from `a` (a 32-row block) and columns from the wave's RW
// tiles of B fragments; only the first NR tiles are formed (a wave whose
// last tiles lie wholly past the rows it owns skips them).
template <typename T, int KS, int RW, int NR = RW>
__device__ inline void logits(f32x4 (&S)[2][RW], const typename Elem<T>::frag (&a)[KS][2],
                              const typename Elem<T>::frag (&b)[RW][KS]) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) S[ct][rt] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int rt = 0; rt < NR; ++rt) S[ct][rt] = Elem<T>::mma(a[s][ct], b[rt][s], S[ct][rt]);
}

// The same products accumulated onto S as given (S holds a bias per logit:
// with keys pre-scaled to log2 units the first MFMA then starts from the
// bias, and no multiply-add is left for the exponent).
template <typename T, int KS, int RW, int NR = RW>
__device__ inline void logits_onto(f32x4 (&S)[2][RW], const typename Elem<T>::frag (&a)[KS][2],
                                   const typename Elem<T>::frag (&b)[RW][KS]) {
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int rt = 0; rt < NR; ++rt) S[ct][rt] = Elem<T>::mma(a[s][ct], b[rt][s], S[ct][rt]);
}

// acc[dp][dt][rt] += v[dp][dt] * pf[rt], rt < NR
template <typename T, int D, int NACC, int RW, int NR = RW>
__device__ inline void weighted_sum(f32x4 (&acc)[NACC][2][RW], const typename Elem<T>::frag (&v)[NACC][2],
                                    const typename Elem<T>::frag (&pf)[RW]) {
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < (D >= 32 ? 2 : 1); ++dt)
#pragma unroll
      for (int rt = 0; rt < NR; ++rt) acc[dp][dt][rt] = Elem<T>::mma(v[dp][dt], pf[rt], acc[dp][dt][rt]);
}

// Row tiles of 16 a wave has to form: those that hold at least one of the
// item's nrows rows (wave-uniform).
template <int RW>
__device__ inline int live_row_tiles(int nrows, int wave) {
  const int n = (nrows - wave * RW * 16 + 15) / 16;
  return n < 0 ? 0 : n > RW ? RW : n;
}

// Call f with the compile-time number of row tiles to form: none when no
// tile holds rows, else all RW, or (ONE) a single tile when only the first
// holds rows.  Without ONE the kernel has one copy of its products: the
// second copy costs k_apply about 70 registers.  (RW > 2 with 1 < n < RW
// forms all RW: padded rows are zero and never stored.)
template <int RW, bool ONE, typename F>
__device__ inline void with_live_tiles(int n, F&& f) {
#if MONARCH_ROWSKIP
  if (n == RW) {
    f(std::integral_constant<int, RW>{});
  } else if (ONE && n == 1) {
    f(std::integral_constant<int, 1>{});
  } else if (n > 0) {
    f(std::integral_constant<int, RW>{});
  }
#else
  (void)n;
  f(std::integral_constant<int, RW>{});
#endif
}

// ------------------------------------------------------------------ k_lse --
// CONTIG: rows are consecutive tokens of a head (only with BCAST keys, where
// the logits do not depend on the column or tile).
//
// With BCAST keys (the first L-step) the log-sum-exp is taken against a fixed
// offset per row instead of a running maximum: m_n = c |q_n| max_c1 |Kbar_c1|
// bounds every logit of row n (Cauchy-Schwarz; knorm holds |Kbar_c1| of the
// rounded keys), so no term exceeds 1 and lse = m_n + log2(sum 2^(x - m_n)).
// That saves the maximum, the rescaling and their dependency chain.  If the
// bound is so loose that a row's sum falls below 2^-60 (very large norms
// with nearly orthogonal q and keys), the workgroup recomputes with the
// running maximum.
//
// PRE (first L-step of the inference forward): the block means are stored
// already multiplied by c = log2(e)/sqrt(d) (k_kbar with cscale = c), so the
// products are logits in log2 units as they stand, knorm holds |c Kbar_c1|,
// and each product starts from -m_n in place of a multiply-add per logit.
template <typename T, int D, int RW, int NW, bool BCAST, bool CONTIG, bool PRE = false>
__device__ __forceinline__ void k_lse_item(const T* __restrict__ q,
                                                                      const T* __restrict__ kt,
                                                                      const float* __restrict__ h2,
                                                                      float* __restrict__ lse, LGeom p,
                                                                      const int* __restrict__ stop_at,
                                                                      int it,
                                                                      const float* __restrict__ knorm, int wi, int wn) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int RB = NW * RW * 16;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  __shared__ __align__(16) T sK[2][kStep * DK];
  __shared__ __align__(16) float sH[2][kStep];
  __shared__ float sRed[NW];

  int bh, g = 0, a2 = 0, nrows;
  long long n0, nstride;
  if (CONTIG) {
    const int logical = xcd_remap(wi, wn);
    bh = logical / p.nrb;
    n0 = static_cast<long long>(logical % p.nrb) * RB;
    nstride = 1;
    nrows = p.N - n0 < RB ? static_cast<int>(p.N - n0) : RB;
  } else {
    ColItem it(p, RB, wi, wn);
    bh = it.bh; g = it.g; a2 = it.a2;
    n0 = static_cast<long long>(it.a1_0) * p.b2 + a2;
    nstride = p.b2;
    nrows = it.nrows;
  }
  if (nrows <= 0) return;
  // heads that stopped iterating earlier keep their last log-sum-exps
  if (stop_at && stop_at[bh] != 0 && stop_at[bh] < it) return;
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const T* qh = q + static_cast<long long>(bh) * p.N * D;
  const int nlive = live_row_tiles<RW>(nrows, wave);  // row tiles past the item's rows are skipped

  const int nst = (p.b1 + kStep - 1) / kStep;
  auto fetch = [&](int st, int buf) {
    const int c1 = st * kStep;
    Dma::issue(sK[buf], ks.k + c1 * ks.kstride, ks.kstride, p.b1 - c1);
    if (!BCAST && wave == NW - 1) dma_floats64(sH[buf], ks.h + static_cast<long long>(c1) * ks.hstride, ks.hstride, p.b1 - c1);
  };
  fetch(0, 0);

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

  if constexpr (BCAST && CONTIG) {
    if (knorm) {
      // max_c1 |Kbar_c1| over the head
      float km = 0.0f;
      for (int i = threadIdx.x; i < p.b1; i += NW * kWave) km = fmaxf(km, knorm[static_cast<long long>(bh) * p.b1 + i]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) km = fmaxf(km, __shfl_xor(km, off));
      if (lane == 0) sRed[wave] = km;
      __syncthreads();
      km = sRed[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) km = fmaxf(km, sRed[w]);
      float mrow[RW], ls[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float sq = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = E::slot(bq[rt][s], j);
            sq = __builtin_fmaf(x, x, sq);
          }
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        // a little above the bound: the MFMA sums in fp32
        mrow[rt] = (PRE ? 1.0f : p.c) * sqrtf(sq) * km * 1.00390625f + 0.00390625f;
        ls[rt] = 0.0f;
      }
      // one 32-key block for the first NR row tiles: masked only where keys
      // run past b1
      auto block = [&](const T* tile, int k0, int c1_0, auto masked, auto nr) {
        constexpr int NR = decltype(nr)::value;
        typename E::frag a[KS][2];
        load_rows<T, DK, KS>(a, tile, k0, l16, G);
        f32x4 S[2][RW];
        if constexpr (PRE) {
#pragma unroll
          for (int rt = 0; rt < NR; ++rt)
            S[0][rt] = S[1][rt] = f32x4{-mrow[rt], -mrow[rt], -mrow[rt], -mrow[rt]};
          logits_onto<T, KS, RW, NR>(S, a, bq);
        } else {
          logits<T, KS, RW, NR>(S, a, bq);
        }
#pragma unroll
        for (int rt = 0; rt < NR; ++rt)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float w = PRE ? fast_exp2(S[j >> 2][rt][j & 3])
                                : fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, -mrow[rt]));
            if constexpr (decltype(masked)::value)
              ls[rt] += c1_0 + 8 * G + j < p.b1 ? w : 0.0f;
            else
              ls[rt] += w;
          }
      };
      for (int st = 0; st < nst; ++st) {
        const int cur = st & 1;
        if (st + 1 < nst) fetch(st + 1, cur ^ 1);
        with_live_tiles<RW, false>(nlive, [&](auto nr) {
#pragma unroll
          for (int half = 0; half < kHalves; ++half) {
            const int k0 = 32 * half;
            const int c1_0 = st * kStep + k0;
            if (c1_0 >= p.b1) break;
            if (c1_0 + 32 > p.b1)
              block(sK[cur], k0, c1_0, std::true_type{}, nr);
            else
              block(sK[cur], k0, c1_0, std::false_type{}, nr);
          }
        });
        __syncthreads();
      }
      bool loose = false;
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        ls[rt] += __shfl_xor(ls[rt], 16);
        ls[rt] += __shfl_xor(ls[rt], 32);
        const int r = (wave * RW + rt) * 16 + l16;
        if (r < nrows && !(ls[rt] >= 8.673617379884035e-19f)) loose = true;  // 2^-60 (or NaN)
      }
      if (!__syncthreads_or(loose)) {
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) {
          const int r = (wave * RW + rt) * 16 + l16;
          if (G == 0 && r < nrows) lse[static_cast<long long>(bh) * p.N + n0 + r * nstride] = mrow[rt] + log2f(ls[rt]);
        }
        return;
      }
      fetch(0, 0);  // the buffers are free: start over with the running maximum
    }
  }

  float m[RW], l[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) { m[rt] = -1e30f; l[rt] = 0.0f; }
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) fetch(st + 1, cur ^ 1);
    with_live_tiles<RW, true>(nlive, [&](auto nr) {
      constexpr int NR = decltype(nr)::value;
#pragma unroll
      for (int half = 0; half < kHalves; ++half) {
        const int k0 = 32 * half;
        const int c1_0 = st * kStep + k0;  // first key of this 32-key block
        if (c1_0 >= p.b1) break;
        // keys past b1 only exist in the last block
        const bool tail = c1_0 + 32 > p.b1;
        typename E::frag a[KS][2];
        load_rows<T, DK, KS>(a, sK[cur], k0, l16, G);
        float bias[8];
        if (!BCAST) {
#pragma unroll
          for (int j = 0; j < 8; ++j) bias[j] = sH[cur][k0 + 8 * G + j];
        }
#if MONARCH_LSE_SCHED_BARRIER
        __builtin_amdgcn_sched_barrier(0);
#endif
        f32x4 S[2][RW];
        logits<T, KS, RW, NR>(S, a, bq);
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            x[j] = PRE ? S[j >> 2][rt][j & 3]
                       : BCAST ? S[j >> 2][rt][j & 3] * p.c : __builtin_fmaf(S[j >> 2][rt][j & 3], p.c, bias[j]);
          if (tail) {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = c1_0 + 8 * G + j < p.b1 ? x[j] : kNegInf;
          }
          float cm = x[0];
#pragma unroll
          for (int j = 1; j < 8; ++j) cm = fmaxf(cm, x[j]);
          const float mn = fmaxf(m[rt], cm);
          float acc = l[rt] * fast_exp2(m[rt] - mn);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc += fast_exp2(x[j] - mn);
          l[rt] = acc;
          m[rt] = mn;
        }
      }
    });
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

// Work items k_lse_item, one per workgroup, or looped over by fewer workgroups
// (nitems > 0); nothing runs once every head has stopped iterating (nstop).
template <typename T, int D, int RW, int NW, bool BCAST, bool CONTIG, bool PRE = false>
__global__ __launch_bounds__(NW * kWave, sizeof(T) != 2 ? 1 : BCAST ? MONARCH_LSE_MINW_BCAST : MONARCH_LSE_MINW) void k_lse(const T* __restrict__ q,
                                                                      const T* __restrict__ kt,
                                                                      const float* __restrict__ h2,
                                                                      float* __restrict__ lse, LGeom p,
                                                                      const int* __restrict__ stop_at = nullptr,
                                                                      int it = 0,
                                                                      const float* __restrict__ knorm = nullptr,
    const int* __restrict__ nstop = nullptr, int nitems = 0) {
  if (nstop && *nstop >= p.BH) return;
  const int wn = nitems > 0 ? nitems : static_cast<int>(gridDim.x);
  for (int wi = blockIdx.x; wi < wn; wi += gridDim.x) {
    if (wi != static_cast<int>(blockIdx.x)) __syncthreads();
    k_lse_item<T, D, RW, NW, BCAST, CONTIG, PRE>(q, kt, h2, lse, p, stop_at, it, knorm, wi, wn);
  }
}

// ------------------------------------------------------------ k_aggregate --
// One workgroup: (bh, g, a2) and a block of CB = NW*RW*16 key blocks c1.
// Qh[c1,:] = sum_(a1 in g) L[a1,c1] q_a1 / sum_(a1 in g) L[a1,c1], computed as
// Qh^T = q^T P over steps of 64 rows a1.  q is staged once: the logits read
// it by rows, the weighted sum by columns (transposing LDS reads); the mass
// beta comes from one more product with a ones fragment, so it sums exactly
// the rounded weights the weighted sum uses.
template <typename T, int D, int RW, int NW, bool BCAST>
__device__ __forceinline__ void k_aggregate_item(const T* __restrict__ q,
                                                          const T* __restrict__ kt,
                                                          const float* __restrict__ h2,
                                                          const float* __restrict__ lse,
                                                          T* __restrict__ qhat, float* __restrict__ beta_out,
                                                          LGeom p, const int* __restrict__ stop_at,
                                                          int it, int wi, int wn) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int CB = NW * RW * 16;
  constexpr int NT = NW * kWave;
  constexpr int NDP = D / 32;  // pairs of 16-wide d tiles (0 when D == 16)
  constexpr int NACC = NDP > 0 ? NDP : 1;
  __shared__ __align__(16) T sQ[2][kStep * DK];
  __shared__ float sL[2][kStep];

  // decode (bh, g, a2, cb)
  const int logical = xcd_remap(wi, wn);
  const int cb = logical % p.nrb;
  int rest = logical / p.nrb;
  const int a2 = rest % p.b2;
  rest /= p.b2;
  const int g = rest % p.t;
  const int bh = rest / p.t;
  const int lo = tile_lo(g, p.b1r, p.t), hi = tile_lo(g + 1, p.b1r, p.t);
  if (stop_at && stop_at[bh] != 0 && stop_at[bh] < it) return;  // head done iterating
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
    // rows c1 >= b1 (zero keys) are computed but never stored: no mask needed
    bias[rt] = BCAST ? 0.0f : (c1 < p.b1 ? ks.bias(c1, p.b1) : 0.0f);
  }

  f32x4 acc[NACC][2][RW];
  f32x4 accb[RW];  // column sums of the rounded weights (the mass beta)
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    accb[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) acc[dp][dt][rt] = f32x4{0, 0, 0, 0};
  }
  const typename E::frag ones = E::ones();

  const T* qh = q + static_cast<long long>(bh) * p.N * D;
  const float* lh = lse + static_cast<long long>(bh) * p.N;
  const long long qstride = static_cast<long long>(p.b2) * D;
  const int nrows = hi - lo;
  const int nst = (nrows + kStep - 1) / kStep;
  TileLoader<T, D, DK, kStep, NT> ld;
  float lpre = 0.0f;
  // sL holds -lse of each staged row (-inf past the tile: weight 0)
  auto fetch = [&](int st) {
    const long long n_first = static_cast<long long>(lo + st * kStep) * p.b2 + a2;
    const int nvalid = nrows - st * kStep;
    ld.load(qh + n_first * D, qstride, nvalid);
    if (threadIdx.x < kStep)
      lpre = static_cast<int>(threadIdx.x) < nvalid
                 ? -lh[n_first + threadIdx.x * static_cast<long long>(p.b2)]
                 : kNegInf;
  };
  fetch(0);
  ld.store(sQ[0]);
  if (threadIdx.x < kStep) sL[0][threadIdx.x] = lpre;
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    const bool more = st + 1 < nst;
    if (more) fetch(st + 1);
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
      const int k0 = 32 * half;
      if (st * kStep + k0 >= nrows) break;
      // all LDS operands of this 32-row block first: rows of q for the
      // logits, columns of q for the weighted sum, and -lse
      typename E::frag a[KS][2];
      typename E::frag v[NACC][2];
      load_rows<T, DK, KS>(a, sQ[cur], k0, l16, G);
      load_cols<T, D, DK, NACC>(v, sQ[cur], k0);
      float nl[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) nl[j] = sL[cur][k0 + 8 * G + j];
      __builtin_amdgcn_sched_barrier(0);
      // S tiles: rows a1 (permuted), columns c1 (the wave's key rows)
      f32x4 S[2][RW];
      logits<T, KS, RW>(S, a, bk);
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, BCAST ? nl[j] : nl[j] + bias[rt]));
        pf[rt] = E::pack(w);
        accb[rt] = E::mma(ones, pf[rt], accb[rt]);
      }
      weighted_sum<T, D, NACC, RW>(acc, v, pf);
    }
    if (more) {
      ld.store(sQ[cur ^ 1]);
      if (threadIdx.x < kStep) sL[cur ^ 1][threadIdx.x] = lpre;
    }
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const float b = accb[rt][0];  // every element of column c1 = l16 holds beta[c1]
    const float inv = b > 0.0f ? 1.0f / b : 0.0f;
    const int c1 = cb * CB + (wave * RW + rt) * 16 + l16;
    if (c1 >= p.b1) continue;
    const long long row = ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2 + a2;
    store_rows<T, D, NACC, RW>(qhat + row * D, acc, rt, inv, G);
    if (beta_out && G == 0) beta_out[row] = b;
  }
}

// Work items k_aggregate_item, one per workgroup, or looped over by fewer workgroups
// (nitems > 0); nothing runs once every head has stopped iterating (nstop).
template <typename T, int D, int RW, int NW, bool BCAST>
__global__ __launch_bounds__(NW * kWave, MONARCH_AGG_MINW) void k_aggregate(const T* __restrict__ q,
                                                          const T* __restrict__ kt,
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
    k_aggregate_item<T, D, RW, NW, BCAST>(q, kt, h2, lse, qhat, beta_out, p, stop_at, it, wi, wn);
  }
}

// ------------------------------------------------------- k_aggregate_col --
// Same result as k_aggregate for tiles of at most kColRows rows: the whole q
// column of the tile and its log-sum-exps are copied to LDS once (DMA), then
// all its 32-row blocks run with no further barrier or wait.
// ALLK: one work item is the whole tile column (bh, g, a2) and each wave takes
// the key tiles wave, wave + NW, ... of all b1 key blocks, so the column is
// copied once for every key block instead of once per 128 keys; otherwise an
// item is (bh, g, a2, 128 key blocks), one key tile per wave.
constexpr int kColRows = 256;
#ifndef MONARCH_AGG_ALLK
#define MONARCH_AGG_ALLK 1
#endif

// PRE: block-mean keys pre-scaled by c (see k_lse); each logit product starts
// from -lse of its row.
template <typename T, int D, int RW, int NW, bool BCAST, bool PRE = false, bool ALLK = false>
__device__ __forceinline__ void k_aggregate_col_item(const T* __restrict__ q,
                                                                                const T* __restrict__ kt,
                                                                                const float* __restrict__ h2,
                                                                                const float* __restrict__ lse,
                                                                                T* __restrict__ qhat,
                                                                                float* __restrict__ beta_out, LGeom p,
                                                                                const int* __restrict__ stop_at,
                                                                                int it, int wi, int wn) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  constexpr int NSTEP = kColRows / kStep;
  __shared__ __align__(16) T sQ[NSTEP][kStep * DK];
  __shared__ __align__(16) float sL[NSTEP][kStep];

  const int logical = xcd_remap(wi, wn);
  const int cb = logical % p.nrb;
  int rest = logical / p.nrb;
  const int a2 = rest % p.b2;
  rest /= p.b2;
  const int g = rest % p.t;
  const int bh = rest / p.t;
  const int lo = tile_lo(g, p.b1r, p.t), hi = tile_lo(g + 1, p.b1r, p.t);
  const int nrows = hi - lo;
  const int nst = (nrows + kStep - 1) / kStep;
  if (stop_at && stop_at[bh] != 0 && stop_at[bh] < it) return;  // head done iterating
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;

  const T* qh = q + static_cast<long long>(bh) * p.N * D;
  const float* lh = lse + static_cast<long long>(bh) * p.N;
  const long long qstride = static_cast<long long>(p.b2) * D;
  for (int st = 0; st < nst; ++st) {
    const long long n_first = static_cast<long long>(lo + st * kStep) * p.b2 + a2;
    const int nvalid = nrows - st * kStep;
    Dma::issue(sQ[st], qh + n_first * D, qstride, nvalid);
    if (wave == NW - 1) dma_floats64(sL[st], lh + n_first, p.b2, nvalid);
  }

  const typename E::frag ones = E::ones();
  __syncthreads();
  // key tiles of RW*16 key blocks: this wave's one (cb * NW + wave), or with
  // ALLK every NW-th; a wave whose key tiles all lie past b1 has nothing to
  // compute or store (it took its share of the column's DMA above)
  const int nkt = (p.b1 + RW * 16 - 1) / (RW * 16);
  const int kt0 = ALLK ? wave : cb * NW + wave;
  const int kt_end = ALLK ? nkt : (kt0 + 1 < nkt ? kt0 + 1 : nkt);
  const int nblk = (nrows + 31) / 32;
  constexpr int kMaxBlk = kColRows / 32;
  // a last block of at most 16 rows takes half the logits and exponentials
  // (bf16): its rows sit in the contraction slots of the first logit half
  constexpr bool kHalfOk = MONARCH_AGG_HALF && PRE && sizeof(T) == 2 && D >= 32;
  const bool half_last = kHalfOk && nrows - 32 * (nblk - 1) <= 16;
  const int nfull = half_last ? nblk - 1 : nblk;
  for (int ktile = kt0; ktile < kt_end; ktile += NW) {
    const int c1base = ktile * RW * 16;
    typename E::frag bk[RW][KS];
    float bias[RW];
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      const int c1 = c1base + rt * 16 + l16;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int col = s * 32 + 8 * G;
        bk[rt][s] = (c1 < p.b1 && col < D) ? E::load(ks.k + c1 * ks.kstride + col) : E::zero();
        // PRE: the keys negated (a sign flip of each bf16), so that the product
        // starts from +lse and ends at lse - x: the exponent's negation is then
        // a free input modifier of v_exp_f32, not one instruction per lse value
        if constexpr (PRE) {
          uint4 u = __builtin_bit_cast(uint4, bk[rt][s]);
          u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
          bk[rt][s] = __builtin_bit_cast(typename E::frag, u);
        }
      }
      bias[rt] = BCAST ? 0.0f : (c1 < p.b1 ? ks.bias(c1, p.b1) : 0.0f);
    }
    f32x4 acc[NACC][2][RW];
    f32x4 accb[RW];
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      accb[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) acc[dp][dt][rt] = f32x4{0, 0, 0, 0};
    }

    // the column's 32-row blocks, unrolled: every LDS address is a per-lane
    // offset plus an immediate, and only the last block masks rows
#pragma unroll
    for (int blk = 0; blk < kMaxBlk; ++blk) {
      if (blk >= nfull) break;
      const int st = blk / kHalves, k0 = 32 * (blk % kHalves);
      const int r0 = 32 * blk;
      const bool tail = r0 + 32 > nrows;
      typename E::frag a[KS][2];
      typename E::frag v[NACC][2];
      load_rows<T, DK, KS>(a, sQ[st], k0, l16, G);
      load_cols<T, D, DK, NACC>(v, sQ[st], k0);
      float lr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) lr[j] = sL[st][k0 + 8 * G + j];
#if MONARCH_AGG_SCHED_BARRIER
      __builtin_amdgcn_sched_barrier(0);
#endif
      f32x4 S[2][RW];
      if constexpr (PRE) {
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) {
          S[0][rt] = f32x4{lr[0], lr[1], lr[2], lr[3]};
          S[1][rt] = f32x4{lr[4], lr[5], lr[6], lr[7]};
        }
        logits_onto<T, KS, RW>(S, a, bk);  // lse - x (negated keys)
      } else {
        logits<T, KS, RW>(S, a, bk);
      }
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[j] = PRE ? fast_exp2(-S[j >> 2][rt][j & 3])
                     : fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, BCAST ? -lr[j] : bias[rt] - lr[j]));
        if (tail) {
          const int lim = nrows - r0 - 8 * G;  // rows of this lane group still in the tile
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = j < lim ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
        accb[rt] = E::mma(ones, pf[rt], accb[rt]);
      }
      weighted_sum<T, D, NACC, RW>(acc, v, pf);
    }
    if constexpr (kHalfOk) {
      if (half_last) {
        // rows r0 .. r0+15 in natural order: logit slot 4G+i is row 4G+i and
        // lands in contraction slot 8G+i; slots 8G+4..7 get weight 0 (and
        // zero values)
        const int st = nfull / kHalves, k0 = 32 * (nfull % kHalves);
        const int r0 = 32 * nfull;
        const T* tile = sQ[st];
        typename E::frag a[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = Tile<T, DK>::load8(tile, k0 + l16, s * 32 + 8 * G);
        typename E::frag v[NACC][2];
#pragma unroll
        for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) v[dp][dt] = Tile<T, DK>::load_tr_half(tile, k0, 32 * dp + 4 * dt, 8);
        float lr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lr[i] = sL[st][k0 + 4 * G + i];
        const int lim = nrows - r0 - 4 * G;
        typename E::frag pf[RW];
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) {
          f32x4 S0 = PRE ? f32x4{lr[0], lr[1], lr[2], lr[3]} : f32x4{0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < KS; ++s) S0 = E::mma(a[s], bk[rt][s], S0);
          float w[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = PRE ? fast_exp2(-S0[i])
                                : fast_exp2(__builtin_fmaf(S0[i], p.c, BCAST ? -lr[i] : bias[rt] - lr[i]));
            w[i] = i < lim ? x : 0.0f;
            w[4 + i] = 0.0f;
          }
          pf[rt] = E::pack(w);
          accb[rt] = E::mma(ones, pf[rt], accb[rt]);
        }
        weighted_sum<T, D, NACC, RW>(acc, v, pf);
      }
    }

#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      const float b = accb[rt][0];
      const float inv = b > 0.0f ? 1.0f / b : 0.0f;
      const int c1 = c1base + rt * 16 + l16;
      if (c1 >= p.b1) continue;
      const long long row = ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2 + a2;
      store_rows<T, D, NACC, RW>(qhat + row * D, acc, rt, inv, G);
      if (beta_out && G == 0) beta_out[row] = b;
    }
  }
}

// Work items k_aggregate_col_item, one per workgroup, or looped over by fewer workgroups
// (nitems > 0); nothing runs once every head has stopped iterating (nstop).
template <typename T, int D, int RW, int NW, bool BCAST, bool PRE = false, bool ALLK = MONARCH_AGG_ALLK>
__global__ __launch_bounds__(NW * kWave, MONARCH_AGG_MINW) void k_aggregate_col(const T* __restrict__ q,
                                                                                const T* __restrict__ kt,
                                                                                const float* __restrict__ h2,
                                                                                const float* __restrict__ lse,
                                                                                T* __restrict__ qhat,
                                                                                float* __restrict__ beta_out, LGeom p,
                                                                                const int* __restrict__ stop_at = nullptr,
                                                                                int it = 0,
    const int* __restrict__ nstop = nullptr, int nitems = 0) {
  if (nstop && *nstop >= p.BH) return;
  const int wn = nitems > 0 ? nitems : static_cast<int>(gridDim.x);
  for (int wi = blockIdx.x; wi < wn; wi += gridDim.x) {
    if (wi != static_cast<int>(blockIdx.x)) __syncthreads();
    k_aggregate_col_item<T, D, RW, NW, BCAST, PRE, ALLK>(q, kt, h2, lse, qhat, beta_out, p, stop_at, it, wi, wn);
  }
}

// ---------------------------------------------------------------- k_apply --
// One workgroup: (bh, g, a2) and a block of RB = NW*RW*16 rows a1 of tile g.
// y[a1,:] = sum_c1 L[a1,c1] U[g,c1,a2,:], with L normalised by the stored
// log-sum-exp (no running rescale), computed as y^T = U^T P^T.
// PRE: block-mean keys pre-scaled by c (see k_lse); each logit product starts
// from -lse of its row.
template <typename T, int D, int RW, int NW, bool BCAST, bool PRE = false>
__global__ __launch_bounds__(NW * kWave, MONARCH_APP_MINW) void k_apply(const T* __restrict__ q,
                                                                        const T* __restrict__ kt,
                                                                        const float* __restrict__ h2,
                                                                        const float* __restrict__ lse,
                                                                        const T* __restrict__ u,
                                                                        T* __restrict__ out, LGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int RB = NW * RW * 16;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  // the two stages' buffers are distinct LDS objects, used in a fixed
  // alternation (see the stage loop): the compiler can then tell that the
  // DMA into one never writes what the other stage reads, and the prefetch
  // overlaps the products instead of being waited for at once
  __shared__ __align__(16) T sK0[kStep * DK];
  __shared__ __align__(16) T sK1[kStep * DK];
  __shared__ __align__(16) T sU0[kStep * DK];
  __shared__ __align__(16) T sU1[kStep * DK];
  __shared__ __align__(16) float sH0[BCAST ? 1 : kStep];
  __shared__ __align__(16) float sH1[BCAST ? 1 : kStep];

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
  const typename Dma::Plan plk = Dma::plan(ks.kstride), plu = Dma::plan(ustride);

  const int nst = (p.b1 + kStep - 1) / kStep;
  auto fetch = [&](int st, T* tK, T* tU, float* tH) {
    const int c1 = st * kStep;
    Dma::issue(tK, ks.k + c1 * ks.kstride, plk, ks.kstride, p.b1 - c1);
    Dma::issue(tU, ucol + c1 * ustride, plu, ustride, p.b1 - c1);
    if (!BCAST && wave == NW - 1) dma_floats64(tH, ks.h + static_cast<long long>(c1) * ks.hstride, ks.hstride, p.b1 - c1);
  };
  fetch(0, sK0, sU0, sH0);

  typename E::frag bq[RW][KS];
  float nlrow[RW];  // -lse of the lane's rows
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    const bool ok = r < it.nrows;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bq[rt][s] = (ok && col < D) ? E::load(qh + (n0 + r * nstride) * D + col) : E::zero();
    }
    nlrow[rt] = ok ? -lh[n0 + r * nstride] : 0.0f;
  }
  f32x4 acc[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) acc[dp][dt][rt] = f32x4{0, 0, 0, 0};
  __syncthreads();

  // row tiles of this wave that hold rows of the item: the others are skipped
  const int nlive = live_row_tiles<RW>(it.nrows, wave);
  // one step's products on (cK, cU, cH) for the first NR row tiles
  auto products_of = [&](int st, const T* cK, const T* cU, const float* cH, auto nr) {
    constexpr int NR = decltype(nr)::value;
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
      const int k0 = 32 * half;
      const int c1_0 = st * kStep + k0;
      if (c1_0 >= p.b1) break;
      // keys past b1 only exist in the last block: weight 0
      const bool tail = c1_0 + 32 > p.b1;
      typename E::frag a[KS][2];
      typename E::frag v[NACC][2];
      load_rows<T, DK, KS>(a, cK, k0, l16, G);
      load_cols<T, D, DK, NACC>(v, cU, k0);
      float bias[8];
      if (!BCAST) {
#pragma unroll
        for (int j = 0; j < 8; ++j) bias[j] = cH[k0 + 8 * G + j];
      }
#if MONARCH_APP_SCHED_BARRIER
      __builtin_amdgcn_sched_barrier(0);
#endif
      f32x4 S[2][RW];
      if constexpr (PRE) {
#pragma unroll
        for (int rt = 0; rt < NR; ++rt)
          S[0][rt] = S[1][rt] = f32x4{nlrow[rt], nlrow[rt], nlrow[rt], nlrow[rt]};
        logits_onto<T, KS, RW, NR>(S, a, bq);
      } else {
        logits<T, KS, RW, NR>(S, a, bq);
      }
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < NR; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[j] = PRE ? fast_exp2(S[j >> 2][rt][j & 3])
                     : fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, BCAST ? nlrow[rt] : bias[j] + nlrow[rt]));
        if (tail) {
          asm volatile("");  // keeps the tail a (wave-uniform) branch: no selects in the other key blocks
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = c1_0 + 8 * G + j < p.b1 ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
      }
      weighted_sum<T, D, NACC, RW, NR>(acc, v, pf);
    }
  };
  // one step: prefetch the next into (nK, nU, nH), products on (cK, cU, cH)
  auto stage = [&](int st, const T* cK, const T* cU, const float* cH, T* nK, T* nU, float* nH) {
    if (st + 1 < nst) fetch(st + 1, nK, nU, nH);
    with_live_tiles<RW, false>(nlive, [&](auto nr) { products_of(st, cK, cU, cH, nr); });
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 2) {
    stage(st, sK0, sU0, sH0, sK1, sU1, sH1);
    if (st + 1 < nst) stage(st + 1, sK1, sU1, sH1, sK0, sU0, sH0);
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
// cscale multiplies the means before they are rounded and stored: 1, or
// c = log2(e)/sqrt(d) for the kernels that take pre-scaled keys (PRE).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_kbar(const T* __restrict__ k, T* __restrict__ kbar,
                                              float* __restrict__ knorm, int BH, int b1, int b2,
                                              float cscale = 1.0f) {
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
  // every lane now holds the sums of its columns; round the means as they
  // are stored and take |Kbar| of the rounded row (the bound k_lse uses)
  const float inv = cscale / static_cast<float>(b2);
  T mean[V];
  float sq = 0.0f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    mean[j] = E::from_f32(acc[j] * inv);
    const float x = E::to_f32(mean[j]);
    sq = __builtin_fmaf(x, x, sq);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) sq += __shfl_xor(sq, off);
  if (ro == 0) {
    T* dst = kbar + item * D + col;
#pragma unroll
    for (int j = 0; j < V; ++j) dst[j] = mean[j];
    if (knorm && lane == 0) knorm[item] = sqrtf(sq);
  }
}

// The same block means for long key blocks (thousands of keys, e.g. a whole
// frame): one workgroup of four waves per block c1, each wave summing every
// fourth group of rows, the four partial sums added in LDS in a fixed order.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_kbar_long(const T* __restrict__ k, T* __restrict__ kbar,
                                                   float* __restrict__ knorm, int b2, float cscale = 1.0f) {
  using E = Elem<T>;
  constexpr int V = E::kVec;
  constexpr int LPR = D / V;        // lanes per row
  constexpr int RPI = kWave / LPR;  // rows per wave and pass
  constexpr int NWV = 4;
  __shared__ float part[NWV][D];
  const long long item = blockIdx.x;  // bh*b1 + c1
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = (lane % LPR) * V, ro = lane / LPR;
  const T* src = k + item * b2 * D;
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.0f;
  for (int c2 = wave * RPI + ro; c2 < b2; c2 += NWV * RPI) {
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
#pragma unroll
    for (int j = 0; j < V; ++j) part[wave][col + j] = acc[j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = ((part[0][col + j] + part[1][col + j]) + part[2][col + j]) + part[3][col + j];
  // round the means as they are stored and take |Kbar| of the rounded row
  const float inv = cscale / static_cast<float>(b2);
  T mean[V];
  float sq = 0.0f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    mean[j] = E::from_f32(acc[j] * inv);
    const float x = E::to_f32(mean[j]);
    sq = __builtin_fmaf(x, x, sq);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) sq += __shfl_xor(sq, off);
  if (ro == 0) {
    T* dst = kbar + item * D + col;
#pragma unroll
    for (int j = 0; j < V; ++j) dst[j] = mean[j];
    if (knorm && lane == 0) knorm[item] = sqrtf(sq);
  }
}

// ------------------------------------------------------------- k_objective --
// After the L-step of iteration `it`: F = sum_n lse_n (nats) is the objective
// of the current factors (the L-step is the exact maximiser).  Per head, one
// workgroup: stop after this iteration when it == max_it, or when it >= 2 and
// the gain over the previous L-step per query token is <= tol.  Heads that
// already stopped are left alone.  The sum runs in double in a fixed order.
// The first L-step leaves out the entropy of the uniform R, log(b2), which is
// the same for every key block (it cancels in the softmax); it is added back
// here so that F_1 is the objective proper.
// (A template only so that every translation unit that launches it shares
// one definition.)
// 1024 threads per head; each thread keeps eight loads in flight (strided
// by the block, so every load instruction of the block is coalesced).
constexpr int kObjThreads = 1024;
template <int kUnused = 0>
__global__ __launch_bounds__(kObjThreads) void k_objective(const float* __restrict__ lse, int N, int b2,
                                                           double* __restrict__ fprev, int* __restrict__ stop_at,
                                                           int it, int max_it, float tol,
                                                           int* __restrict__ nstop_upto) {
  constexpr int U = 8;
  const int bh = blockIdx.x;
  if (stop_at[bh] != 0) return;
  __shared__ double red[kObjThreads];
  double acc = 0.0;
  const float* l = lse + static_cast<long long>(bh) * N;
  int n = threadIdx.x;
  for (; n + (U - 1) * kObjThreads < N; n += U * kObjThreads) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = l[n + u * kObjThreads];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += static_cast<double>(x[u]);
  }
  for (; n < N; n += kObjThreads) acc += static_cast<double>(l[n]);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = kObjThreads / 2; off > 0; off >>= 1) {
    if (static_cast<int>(threadIdx.x) < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double F = red[0] * 0.69314718055994530942;  // log2 units -> nats
    if (it == 1) F += static_cast<double>(N) * log(static_cast<double>(b2));
    const bool stop = it >= max_it || (it >= 2 && F - fprev[bh] <= static_cast<double>(tol) * N);
    fprev[bh] = F;
    if (stop) {
      stop_at[bh] = it;
      // nstop_upto[i] counts the heads stopped after iteration <= i; once
      // nstop_upto[it - 1] reaches BH every launch of iteration it returns at once
      for (int i = it; i <= max_it; ++i) atomicAdd(nstop_upto + i, 1);
    }
  }
}

template <int kUnused = 0>
__global__ __launch_bounds__(256) void k_fill_int(int* __restrict__ p, int n, int value) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = value;
}

}  // namespace monarch
