// Backward of the R-step for long key blocks (b2 > 128, e.g. blocks of whole
// frames): the part that kb_rside_a computes per row (g, c1, a2) when a whole
// block row fits one wave.  Here the block's keys stream through LDS 64 at a
// time, once: the row statistics need no pass of their own.
//   lse: the training forward's long R-step stored each row's log-sum-exp;
//   rho = <R, dR'> is a product of stored rows (as FlashAttention takes
//   sum_j P dP from O and dO): for the last R-step dR = <dU, v_c2> and
//   sum_c2 R dR = <dU, U>; for an earlier one dR' = <dKt, k_c2> - dhl (x - lse)
//   (dhl = dH ln 2, x the logit in log2 units) and
//   sum_c2 R dR' = <dKt, Kt> + dhl H, with Kt = sum R k and H in bits, both
//   stored by the forward.
// Then per step R = 2^(x - lse), dz = R (dR' - rho), dQh += sum_c2 dz k_c2,
// and at the end G = s dQh / beta and e = <G, Qh>.  It stores G, e and the
// row statistics (lse, rho) as kb_rside_a does, for kb_rside_b, which takes
// the keys of a long block in slices of 128.
#pragma once

#include "backward.h"

namespace monarch {

struct RBLGeom {
  int BH, b1, b2, t;
  int nrb;  // blocks of 32*NW rows a2 per (key block, tile)
  float c;  // log2(e) / sqrt(d)
  float s;  // 1 / sqrt(d)
};

template <typename T, int D, int NW, bool MID>
__global__ __launch_bounds__(NW * kWave) void kb_rside_a_long(const T* __restrict__ k, const T* __restrict__ v,
                                                              const T* __restrict__ qhat, const T* __restrict__ du,
                                                              const float* __restrict__ dh,
                                                              const float* __restrict__ beta,
                                                              const float* __restrict__ rl,  // the rows' lse (log2)
                                                              const T* __restrict__ ux,      // U, or Kt (MID)
                                                              const float* __restrict__ hx,  // H in bits (MID)
                                                              T* __restrict__ gq, float* __restrict__ ev,
                                                              float* __restrict__ lser, float* __restrict__ rho,
                                                              RBLGeom p) {
  using E = Elem<T>;
  constexpr int RW = 2;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  constexpr int RB = NW * RW * 16;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  // two stages of K (and V, which an earlier R-step does not need: its
  // cotangent pairs with k) as distinct LDS objects
  __shared__ __align__(16) T sK0[kStep * DK];
  __shared__ __align__(16) T sK1[kStep * DK];
  __shared__ __align__(16) T sV0[MID ? 8 : kStep * DK];
  __shared__ __align__(16) T sV1[MID ? 8 : kStep * DK];

  const int item = xcd_remap(blockIdx.x, gridDim.x);  // ((bh*b1 + c1)*t + g)*nrb + rb
  const int rb = item % p.nrb;
  int rest = item / p.nrb;
  const int g = rest % p.t;
  rest /= p.t;
  const int c1 = rest % p.b1;
  const int bh = rest / p.b1;
  const long long kblk = (static_cast<long long>(bh) * p.b1 + c1) * p.b2 * D;
  const long long rbase = ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2;  // row a2 = 0
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const int nst = (p.b2 + kStep - 1) / kStep;
  auto fetch = [&](int st, T* tK, T* tV) {
    const int c2 = st * kStep;
    Dma::issue(tK, k + kblk + static_cast<long long>(c2) * D, D, p.b2 - c2);
    if (!MID) Dma::issue(tV, v + kblk + static_cast<long long>(c2) * D, D, p.b2 - c2);
  };
  fetch(0, sK0, sV0);

  // per row tile: the aggregated query and the cotangent as B operands, and
  // the row statistics
  typename E::frag bq[RW][KS], bd[RW][KS];
  float lse2[RW], rh[RW], dhl[RW];
  bool row_ok[RW];
  long long row[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int a2 = rb * RB + (wave * RW + rt) * 16 + l16;
    row_ok[rt] = a2 < p.b2;
    row[rt] = rbase + (row_ok[rt] ? a2 : 0);
    typename E::frag bx[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      const bool ok = row_ok[rt] && col < D;
      bq[rt][s] = ok ? E::load(qhat + row[rt] * D + col) : E::zero();
      bd[rt][s] = ok ? E::load(du + row[rt] * D + col) : E::zero();
      bx[s] = ok ? E::load(ux + row[rt] * D + col) : E::zero();
    }
    float r0 = dot_frags<T, KS>(bd[rt], bx);
    r0 += __shfl_xor(r0, 16);
    r0 += __shfl_xor(r0, 32);
    dhl[rt] = MID ? (row_ok[rt] ? dh[row[rt]] * kLn2 : 0.0f) : 0.0f;
    lse2[rt] = row_ok[rt] ? rl[row[rt]] : 0.0f;
    rh[rt] = MID ? r0 + dhl[rt] * (row_ok[rt] ? hx[row[rt]] : 0.0f) : r0;
  }
  f32x4 acc[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) acc[dp][0][rt] = acc[dp][1][rt] = f32x4{0, 0, 0, 0};
  __syncthreads();

  auto stage = [&](int st, const T* cK, const T* cV, T* nK, T* nV) {
    if (st + 1 < nst) fetch(st + 1, nK, nV);
    const int c2s = st * kStep;
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
      if (c2s + 32 * h >= p.b2) break;
      typename E::frag a[KS][2];
      f32x4 S[2][RW], DR[2][RW];
      // dR - rho: the products start from -rho
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) DR[0][rt] = DR[1][rt] = f32x4{-rh[rt], -rh[rt], -rh[rt], -rh[rt]};
      load_rows<T, DK, KS>(a, cK, 32 * h, l16, G);
      logits<T, KS, RW>(S, a, bq);
      if (MID) {
        products<T, KS, RW>(DR, a, bd);  // + <dKt, k>
      } else {
        load_rows<T, DK, KS>(a, cV, 32 * h, l16, G);
        products<T, KS, RW>(DR, a, bd);  // + <dU, v>
      }
      // keys past b2 exist only in the block's last 32-key half
      const bool tail = c2s + 32 * h + 32 > p.b2;
      typename E::frag zf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float z[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xl = __builtin_fmaf(S[j >> 2][rt][j & 3], p.c, -lse2[rt]);  // log2 R
          float dr = DR[j >> 2][rt][j & 3];
          if (MID) dr = __builtin_fmaf(-dhl[rt], xl, dr);
          z[j] = fast_exp2(xl) * dr;
        }
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j) z[j] = c2s + 32 * h + 8 * G + j < p.b2 ? z[j] : 0.0f;
        }
        zf[rt] = E::pack(z);
      }
      // dQh^T = K^T dz^T: rows d, columns a2
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, cK, 32 * h);
      weighted_sum<T, D, NACC, RW>(acc, vv, zf);
    }
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 2) {
    stage(st, sK0, sV0, sK1, sV1);
    if (st + 1 < nst) stage(st + 1, sK1, sV1, sK0, sV0);
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const float bt = row_ok[rt] ? beta[row[rt]] : 0.0f;
    const float sc = bt > 0.0f ? p.s / bt : 0.0f;
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) {
      acc[dp][0][rt] *= sc;
      acc[dp][1][rt] *= sc;
    }
    // e = <G, Qh> with the rounded Qh the forward used (held in bq: its
    // lane slots are the accumulator's d positions)
    float e;
    if constexpr (D >= 32)
      e = dot_acc_frags<T, NACC, RW>(bq[rt], acc, rt);
    else
      e = dot_acc_row<T, D, NACC, RW>(qhat + row[rt] * D, acc, rt, G);
    e += __shfl_xor(e, 16);
    e += __shfl_xor(e, 32);
    if (row_ok[rt]) {
      store_rows<T, D, NACC, RW>(gq + row[rt] * D, acc, rt, 1.0f, G);
      if (G == 0) {
        ev[row[rt]] = e;
        lser[row[rt]] = lse2[rt];
        rho[row[rt]] = rh[rt];
      }
    }
  }
}

}  // namespace monarch
