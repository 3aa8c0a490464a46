// R-side kernel for long key blocks (b2 > 128): the same R-step as rside.h,
//   R[g,c1,a2,:] = softmax_c2( s<Qh[g,c1,a2], k_(c1,c2)> ),
//   last iteration:  U[g,c1,a2,:]  = sum_c2 R v_(c1,c2)
//   otherwise:       Kt[g,c1,a2,:] = sum_c2 R k_(c1,c2),  H[g,c1,a2] = -sum_c2 R log2 R
// (yunpan.plus MonarchRT article, "Monarch matrices" and "Innovation 2").
// Blocks this long arise when a block spans a whole frame, b1 = f frames and
// b2 = h*w positions: the spatio-temporal factorisation the VMonarch abstract
// names (inter-frame mixing in L, intra-frame mixing in R).
//
// A block row no longer fits one wave's registers, so the softmax over c2 is
// taken online, as in FlashAttention: one workgroup owns (bh, c1, g) and RB
// rows a2, and the b2 keys (and values) of block c1 stream through LDS 64 at a
// time by double-buffered DMA.  Per row the running maximum m (log2 units),
// the running sum l = sum 2^(x - m) and, for the entropy, the running
// sx = sum 2^(x - m) (x - m) are kept; when m rises to m' they become
//   l' = a l,   sx' = a (sx - (m' - m) l),   acc' = a acc,   a = 2^(m - m'),
// which is the entropy taken online alongside the block softmax (the fused
// "online entropy" of the VMonarch abstract).  At the end U (or Kt) = acc / l
// and H in bits = log2 l - sx / l; a training forward also keeps each row's
// log-sum-exp m + log2 l for the backward.
#pragma once

#include "lside.h"

namespace monarch {

// Key blocks up to this length use the register-resident R-step (rside.h).
constexpr int kShortB2 = 128;

struct RLGeom {
  int BH, b1, b2, t;
  int nrb;  // blocks of RB rows a2 per (key block, tile)
  float c;  // log2(e) / sqrt(d)
};

// F32SUM (the training forward, which keeps each row's log-sum-exp for the
// backward): the row sum l is taken in fp32 over the unrounded weights, so
// that the backward's recomputed R = 2^(x - lse) sums to 1; otherwise it is
// the MFMA sum of the rounded weights the products use.
template <typename T, int D, int RW, int NW, bool LAST, bool F32SUM = false>
__device__ __forceinline__ void rstep_long_body(const T* __restrict__ k, const T* __restrict__ v,
                                                T* qhat,  // [BH][t][b1][b2][D]; U written over it when LAST
                                                T* __restrict__ ktil, float* __restrict__ hent,
                                                T* uout,  // U goes here instead when not NULL
                                                float* rlse,  // the rows' log-sum-exps (log2), when not NULL
                                                const RLGeom& p, int item, T* sK0, T* sK1, T* sV0, T* sV1) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int RB = NW * RW * 16;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  constexpr float kMaskLogit = -1e30f;

  // item = ((bh * b1 + c1) * t + g) * nrb + rb: the row blocks and tiles of
  // one key block are neighbours, so its K and V blocks are shared in L2
  const int rb = item % p.nrb;
  int rest = item / p.nrb;
  const int g = rest % p.t;
  rest /= p.t;
  const int c1 = rest % p.b1;
  const int bh = rest / p.b1;
  const int a2_0 = rb * RB;
  const int nrows = p.b2 - a2_0 < RB ? p.b2 - a2_0 : RB;
  const long long qbase = ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2 + a2_0;
  const long long kblk = (static_cast<long long>(bh) * p.b1 + c1) * p.b2 * D;

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const int nst = (p.b2 + kStep - 1) / kStep;
  // the lanes' DMA offsets within a 64-key tile, formed once (K and V tiles
  // have the same layout): only the last, partial tile clamps rows per lane
  const typename Dma::Plan plan = Dma::plan(D);
  auto fetch = [&](int st, T* tK, T* tV) {
    const int c2 = st * kStep;
    Dma::issue(tK, k + kblk + static_cast<long long>(c2) * D, plan, D, p.b2 - c2);
    if (LAST) Dma::issue(tV, v + kblk + static_cast<long long>(c2) * D, plan, D, p.b2 - c2);
  };
  fetch(0, sK0, sV0);

  typename E::frag bq[RW][KS];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    const bool ok = r < nrows;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bq[rt][s] = (ok && col < D) ? E::load(qhat + (qbase + r) * D + col) : E::zero();
    }
  }
  // PRES (the bf16 forms without F32SUM): the queries are held pre-scaled by
  // c and every logit product starts from -m, so the products give
  // x' = c<q,k> - m, the exponent's argument itself: no multiply-add per
  // weight.  The training forward (F32SUM) keeps the plain products, the
  // form from which the backward recomputes R.
  constexpr bool PRES = sizeof(T) == 2 && !F32SUM;
  if constexpr (PRES) {
#pragma unroll
    for (int rt = 0; rt < RW; ++rt)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = p.c * E::slot(bq[rt][s], j);
        bq[rt][s] = E::pack(w);
      }
  }
  f32x4 acc[NACC][2][RW];
  // m: the reference maximum of the row (log2 units); accl: the row sum of
  // the rounded weights, summed by an MFMA against a ones fragment (every
  // lane holds its row's whole sum); sx: the lane's share of sum w (x - m)
  f32x4 accl[RW];
  float m[RW], sx[RW], l32[RW];  // l32: F32SUM's lane share of the row sum
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    m[rt] = PRES ? 0.0f : kMaskLogit;  // PRES: the first step sets it
    sx[rt] = 0.0f;
    l32[rt] = 0.0f;
    accl[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) acc[dp][0][rt] = acc[dp][1][rt] = f32x4{0, 0, 0, 0};
  }
  const typename E::frag ones = E::ones();
  __syncthreads();

  // one step of 64 keys: prefetch the next into (nK, nV), products on (cK, cV).
  // The reference maximum moves only when the step's maximum exceeds it by
  // more than kRescale (log2 units), so weights stay below 2^kRescale and the
  // accumulators are rescaled only on those rare steps (one branch for the
  // wave); the logit scale c rides in the exponent's multiply-add (or, with
  // PRES, in the queries).
  constexpr float kRescale = 8.0f;
  constexpr float kBig = 18446744073709551616.0f;  // 2^64, the PRES forms' bound on a half's row sum
  auto stage = [&](int st, const T* cK, const T* cV, T* nK, T* nV) {
    if (st + 1 < nst) fetch(st + 1, nK, nV);
    const int c2s = st * kStep;
    // logits of both 32-key halves (lane: keys 8G + j of each half, row l16
    // of each row tile): raw, or with PRES c<q,k> - m; keys past b2 masked
    f32x4 S[kHalves][2][RW];
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
      typename E::frag a[KS][2];
      load_rows<T, DK, KS>(a, cK, 32 * h, l16, G);
      if constexpr (PRES) {
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) S[h][0][rt] = S[h][1][rt] = f32x4{-m[rt], -m[rt], -m[rt], -m[rt]};
        logits_onto<T, KS, RW>(S[h], a, bq);
      } else {
        logits<T, KS, RW>(S[h], a, bq);
      }
    }
    if (c2s + kStep > p.b2) {
      // only the last step holds keys past b2; the empty asm keeps this a
      // (wave-uniform) branch instead of selects in every step
      asm volatile("");
#pragma unroll
      for (int rt = 0; rt < RW; ++rt)
#pragma unroll
        for (int h = 0; h < kHalves; ++h)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c2s + 32 * h + 8 * G + j >= p.b2) S[h][j >> 2][rt][j & 3] = kMaskLogit;
    }
    if constexpr (PRES) {
      // The reference starts at the first step's maximum (m = 0 before it)
      // and afterwards moves only when a 32-key half's row sum exceeds 2^64
      // (kBig): the sums come from the MFMA the row sums need anyway, and an
      // overflowed weight makes them infinite, so no later step takes a
      // maximum unless its half trips that test.  Weights up to 2^64 lose
      // nothing in bf16 or in the fp32 sums (both keep fp32's exponent
      // range), and the sums of a row stay far below fp32's limit.
      if (st == 0) {
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) {
          float mx = kMaskLogit;
#pragma unroll
          for (int h = 0; h < kHalves; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) mx = fmaxf(mx, S[h][j >> 2][rt][j & 3]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          m[rt] = mx;
#pragma unroll
          for (int h = 0; h < kHalves; ++h) {
            S[h][0][rt] -= mx;
            S[h][1][rt] -= mx;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kHalves; ++h) {
        typename E::frag pf[RW];
        float w[RW][8];
        f32x4 hs[RW];
        auto weights = [&](int rt) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[rt][j] = fast_exp2(S[h][j >> 2][rt][j & 3]);
          pf[rt] = E::pack(w[rt]);
          hs[rt] = E::mma(ones, pf[rt], f32x4{0, 0, 0, 0});
        };
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) weights(rt);
        bool big = false;
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) big = big || !(hs[rt][0] <= kBig);
        if (__any(big)) {
          // rare: the rows whose half sum tripped move the reference up to
          // the half's maximum; their sums and accumulators are rescaled and
          // the half's weights made again
#pragma unroll
          for (int rt = 0; rt < RW; ++rt) {
            float mx = kMaskLogit;
#pragma unroll
            for (int j = 0; j < 8; ++j) mx = fmaxf(mx, S[h][j >> 2][rt][j & 3]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float dm = !(hs[rt][0] <= kBig) ? mx : 0.0f;
            const float a = fast_exp2(-dm);
            if (!LAST) sx[rt] = a * (sx[rt] - dm * 0.25f * accl[rt][0]);
            accl[rt] *= a;
#pragma unroll
            for (int dp = 0; dp < NACC; ++dp) {
              acc[dp][0][rt] *= a;
              acc[dp][1][rt] *= a;
            }
            m[rt] += dm;
#pragma unroll
            for (int h2 = h; h2 < kHalves; ++h2) {
              S[h2][0][rt] -= dm;
              S[h2][1][rt] -= dm;
            }
            weights(rt);
          }
        }
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) {
          accl[rt] += hs[rt];
          if (!LAST) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sx[rt] = __builtin_fmaf(w[rt][j], S[h][j >> 2][rt][j & 3], sx[rt]);
          }
        }
        // X^T P^T (X = V, or K for the next keys): rows d, columns a2
        typename E::frag vv[NACC][2];
        load_cols<T, D, DK, NACC>(vv, LAST ? cV : cK, 32 * h);
        weighted_sum<T, D, NACC, RW>(acc, vv, pf);
      }
    } else {
    bool jump = false;
    float mstep[RW];
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      float mx = kMaskLogit;
#pragma unroll
      for (int h = 0; h < kHalves; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, S[h][j >> 2][rt][j & 3]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mstep[rt] = mx * p.c;  // c > 0: the maximum of the scaled logits
      jump = jump || mstep[rt] > m[rt] + kRescale;
    }
    if (__any(jump)) {
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        const float mnew = mstep[rt] > m[rt] + kRescale ? mstep[rt] : m[rt];
        const float a = fast_exp2(m[rt] - mnew);
        // the row sum is shared by the row's four lane groups: each takes a
        // quarter of the correction of the lane-split entropy sum
        if (!LAST) sx[rt] = a * (sx[rt] - (mnew - m[rt]) * (F32SUM ? l32[rt] : 0.25f * accl[rt][0]));
        if (F32SUM)
          l32[rt] *= a;
        else
          accl[rt] *= a;
        m[rt] = mnew;
#pragma unroll
        for (int dp = 0; dp < NACC; ++dp) {
          acc[dp][0][rt] *= a;
          acc[dp][1][rt] *= a;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float dx = __builtin_fmaf(S[h][j >> 2][rt][j & 3], p.c, -m[rt]);
          w[j] = fast_exp2(dx);
          if (F32SUM) l32[rt] += w[j];
          if (!LAST) sx[rt] = __builtin_fmaf(w[j], dx, sx[rt]);
        }
        pf[rt] = E::pack(w);
        if (!F32SUM) accl[rt] = E::mma(ones, pf[rt], accl[rt]);
      }
      // X^T P^T (X = V, or K for the next keys): rows d, columns a2
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, LAST ? cV : cK, 32 * h);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    }
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 2) {
    stage(st, sK0, sV0, sK1, sV1);
    if (st + 1 < nst) stage(st + 1, sK1, sV1, sK0, sV0);
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    float lt = accl[rt][0];
    if (F32SUM) {
      lt = l32[rt];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
    }
    float st = sx[rt];
    if (!LAST) {
      // the entropy sum over the row's four lane groups (all lanes take part)
      st += __shfl_xor(st, 16);
      st += __shfl_xor(st, 32);
    }
    const int r = (wave * RW + rt) * 16 + l16;
    if (r >= nrows) continue;
    const long long row = qbase + r;
    T* dst = (LAST ? (uout ? uout : qhat) : ktil) + row * D;
    store_rows<T, D, NACC, RW>(dst, acc, rt, 1.0f / lt, G);
    if (!LAST && G == 0) hent[row] = log2f(lt) - st / lt;
    if (rlse && G == 0) rlse[row] = m[rt] + log2f(lt);
  }
}

// LDS of the long R-step: two stages of K (and V for the last R-step) as
// distinct objects, so that each stage's prefetch overlaps the other's products.
#define MONARCH_RSTEP_LONG_LDS(T, DK, WITH_V)                  \
  __shared__ __align__(16) T sK0[kStep * (DK)];                \
  __shared__ __align__(16) T sK1[kStep * (DK)];                \
  __shared__ __align__(16) T sV0[(WITH_V) ? kStep * (DK) : 8]; \
  __shared__ __align__(16) T sV1[(WITH_V) ? kStep * (DK) : 8];

template <typename T, int D, int RW, int NW, bool LAST, bool F32SUM = false>
__global__ __launch_bounds__(NW * kWave) void k_rstep_long(const T* __restrict__ k, const T* __restrict__ v, T* qhat,
                                                           T* __restrict__ ktil, float* __restrict__ hent, T* uout,
                                                           float* __restrict__ rlse, RLGeom p) {
  MONARCH_RSTEP_LONG_LDS(T, (D < 32 ? 32 : D), LAST)
  rstep_long_body<T, D, RW, NW, LAST, F32SUM>(k, v, qhat, ktil, hent, uout, rlse, p, xcd_remap(blockIdx.x, gridDim.x), sK0,
                                      sK1, sV0, sV1);
}

// Iteration `it` of a run that stops each head on its own (stop_at as for
// k_rstep_adaptive): heads that stopped earlier are skipped, a head that stops
// now gets R V, the others the next L-step's keys and entropies.  The
// workgroups loop over nitems work items and return at once when every head
// has stopped (nstop).
template <typename T, int D, int RW, int NW>
__global__ __launch_bounds__(NW * kWave) void k_rstep_long_adaptive(const T* __restrict__ k, const T* __restrict__ v,
                                                                    T* qhat, T* __restrict__ ktil,
                                                                    float* __restrict__ hent,
                                                                    const int* __restrict__ stop_at, int it,
                                                                    RLGeom p, const int* __restrict__ nstop,
                                                                    int nitems) {
  MONARCH_RSTEP_LONG_LDS(T, (D < 32 ? 32 : D), true)
  if (*nstop >= p.BH) return;
  for (int wi = blockIdx.x; wi < nitems; wi += gridDim.x) {
    if (wi != static_cast<int>(blockIdx.x)) __syncthreads();
    const int item = xcd_remap(wi, nitems);
    const int bh = item / (p.nrb * p.t * p.b1);
    const int sa = stop_at[bh];
    if (sa != 0 && sa < it) continue;
    if (sa == it)
      rstep_long_body<T, D, RW, NW, true>(k, v, qhat, nullptr, nullptr, nullptr, nullptr, p, item, sK0, sK1, sV0,
                                          sV1);
    else
      rstep_long_body<T, D, RW, NW, false>(k, v, qhat, ktil, hent, nullptr, nullptr, p, item, sK0, sK1, sV0, sV1);
  }
}

#undef MONARCH_RSTEP_LONG_LDS

}  // namespace monarch
