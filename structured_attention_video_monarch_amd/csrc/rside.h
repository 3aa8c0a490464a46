// R-side kernel: everything indexed by a key block c1 (b2 consecutive tokens).
//
// For one (batch*head, c1) and every tile g the R block is
//   R[g,c1,a2,:] = softmax_c2( s<Qh[g,c1,a2], k_(c1,c2)> ),   a2, c2 in [b2]
// (the R-step of MonarchAttention; yunpan.plus MonarchRT article, section
// "Monarch matrices", Fig. 3; one R per tile: "Innovation 2: tiled Monarch").
// It is consumed at once and never stored:
//   last iteration:  U[g,c1,a2,:]  = sum_c2 R v_(c1,c2)   (written over Qh)
//   otherwise:       Kt[g,c1,a2,:] = sum_c2 R k_(c1,c2)   and the row entropy
//                    H[g,c1,a2] = -sum_c2 R log2 R (in bits), the keys and bias
//                    of the next L-step (the entropy computed alongside the
//                    block softmax, as in the VMonarch abstract's fused
//                    "online entropy").
// The K and V blocks are contiguous (b2 x d) and staged in LDS once per
// workgroup; each wave owns 16 rows a2 and all tiles are looped in-kernel.
#pragma once

#include "device_common.h"

namespace monarch {

struct RGeom {
  int BH, b1, b2, t;
  int b2p;    // b2 rounded up to 32
  float c;    // log2(e) / sqrt(d)
};

// Dynamic LDS bytes: the K block and the V block (last iteration only), both
// swizzled tiles of b2p rows.  The products with R read them by columns
// through transposing LDS reads; K serves both the logits and the next keys.
template <typename T>
inline size_t rside_lds_bytes(int D, int b2p, bool last) {
  return sizeof(T) * static_cast<size_t>(b2p) * (D < 32 ? 32 : D) * (last ? 2 : 1);
}

// Tiles whose aggregated queries one wave loads together (bf16), for the
// last R-step and for the ones before it (which also form the entropy).
#ifndef MONARCH_RSTEP_TB
#define MONARCH_RSTEP_TB 2
#endif
#ifndef MONARCH_RSTEP_TB_MID
#define MONARCH_RSTEP_TB_MID 1
#endif

template <typename T, int D, bool LAST>
__device__ __forceinline__ void rstep_body(const T* __restrict__ k, const T* __restrict__ v,
                                           T* qhat,   // [BH][t][b1][b2][D]; U written over it when LAST
                                           T* __restrict__ ktil, float* __restrict__ hent,
                                           T* uout,   // U goes here instead when not NULL
                                           const RGeom& p, int item) {  // item = bh*b1 + c1
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  using TL = Tile<T, DK>;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  constexpr int MAXCP = 4;  // b2 <= 128
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* sK = reinterpret_cast<T*>(smem_raw);
  T* sV = sK + p.b2p * DK;

  const int c1 = item % p.b1;
  const int bh = item / p.b1;
  const long long blk = static_cast<long long>(item) * p.b2 * D;  // first element of block c1

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const int a2 = wave * 16 + l16;
  const bool row_ok = a2 < p.b2;
  const int ncp = p.b2p / 32;
  auto qrow = [&](int g) { return ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2 + a2; };

  // K (and V) blocks by global->LDS DMA: rows past b2 are copies of row b2-1,
  // whose logits are masked below (weight 0)
  {
    constexpr int ROWB = DK * static_cast<int>(sizeof(T));
    const int nins = p.b2p * ROWB / 1024;
    const int nw = blockDim.x / kWave;
    for (int ci = wave; ci < nins; ci += nw) {
      const int byte = ci * 1024 + 16 * lane;
      const int r = byte / ROWB;
      const int c = ((byte % ROWB) / 16) ^ TL::swz(r);
      int col = c * E::kVec;
      if (col >= D) col -= D;
      const long long src = blk + static_cast<long long>(r < p.b2 ? r : p.b2 - 1) * D + col;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(k + src),
                                       (__attribute__((address_space(3))) void*)(sK + ci * (1024 / static_cast<int>(sizeof(T)))),
                                       16, 0, 0);
      if (LAST)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(v + src),
                                         (__attribute__((address_space(3))) void*)(sV + ci * (1024 / static_cast<int>(sizeof(T)))),
                                         16, 0, 0);
    }
  }
  // aggregated queries of up to TB tiles in flight at once
  constexpr int TB = sizeof(T) == 2 ? (LAST ? MONARCH_RSTEP_TB : MONARCH_RSTEP_TB_MID) : 1;
  typename E::frag bq[TB][KS];
  auto load_query = [&](int i, int g) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      bq[i][s] = (g < p.t && row_ok && col < D) ? E::load(qhat + qrow(g) * D + col) : E::zero();
    }
  };
#pragma unroll
  for (int i = 0; i < TB; ++i) load_query(i, i);
  __syncthreads();
  const T* sX = LAST ? sV : sK;

  for (int g0 = 0; g0 < p.t; g0 += TB) {
#pragma unroll
  for (int gi = 0; gi < TB; ++gi) {
    const int g = g0 + gi;
    if (g >= p.t) break;
    const long long row = qrow(g);
    // logits, transposed: rows c2 (permuted within 32-blocks), columns a2
    f32x4 S[MAXCP][2];
#pragma unroll
    for (int cp = 0; cp < MAXCP; ++cp) {
      S[cp][0] = f32x4{0, 0, 0, 0};
      S[cp][1] = f32x4{0, 0, 0, 0};
      if (cp < ncp) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const typename E::frag a = TL::load8(sK, 32 * cp + perm_row(ct, l16), s * 32 + 8 * G);
            S[cp][ct] = E::mma(a, bq[gi][s], S[cp][ct]);
          }
      }
    }
    // this slot's queries are consumed: load the tile TB further on into it,
    // so that the loads run under this tile's softmax, products and stores
    // (U is written over Q-hat only for the rows of tile g itself)
    if (g + TB < p.t) load_query(gi, g + TB);
    // softmax over c2 for column a2: lane holds c2 = 32cp + 8G + j.  Keys
    // past b2 get the finite logit kMaskLogit: 2^(x - m) is exactly 0 for
    // them and x * 0 stays 0 in the entropy sum below.
    constexpr float kMaskLogit = -1e30f;
    float x[MAXCP][8];
    float mx = kMaskLogit;
#pragma unroll
    for (int cp = 0; cp < MAXCP; ++cp)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c2 = 32 * cp + 8 * G + j;
        x[cp][j] = (cp < ncp && c2 < p.b2) ? S[cp][j >> 2][j & 3] * p.c : kMaskLogit;
        mx = fmaxf(mx, x[cp][j]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // sum of 2^(x - mx) and, for the entropy, of 2^(x - mx) (x - mx);
    // sum_c2 R (x - mx) is their ratio.  Both are taken in one pass, as each
    // exponential is made, so that none of them stays live.
    float sum = 0.0f, sumx = 0.0f;
#pragma unroll
    for (int cp = 0; cp < MAXCP; ++cp)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float dx = x[cp][j] - mx;
        const float e = fast_exp2(dx);
        sum += e;
        if (!LAST) sumx = __builtin_fmaf(e, dx, sumx);
      }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    const float lsum = log2f(sum);
    const float lse2 = mx + lsum;
    // entropy in bits (the unit of the L-step's log2 logits), taken about
    // the row maximum so that no large terms cancel when the logits are
    // large: H2 = log2(sum 2^x) - sum R x = log2(sum 2^(x - mx)) -
    // sum R (x - mx) = H / ln 2, with sum R (x - mx) = sumx / sum.  It is
    // finished here, and the barrier keeps the compiler from sinking the sum
    // to the store below (which would keep every exponential live across the
    // products)
    float h2 = 0.0f;
    if (!LAST) {
      sumx += __shfl_xor(sumx, 16);
      sumx += __shfl_xor(sumx, 32);
      h2 = lsum - sumx / sum;
      __builtin_amdgcn_sched_barrier(0);
    }
    typename E::frag pf[MAXCP];
#pragma unroll
    for (int cp = 0; cp < MAXCP; ++cp) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = fast_exp2(x[cp][j] - lse2);
      pf[cp] = E::pack(w);
    }
    // X^T P^T (X = V, or K for the next keys): rows d, columns a2
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[NACC][2][1];
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) {
      acc[dp][0][0] = f32x4{0, 0, 0, 0};
      acc[dp][1][0] = f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int cp = 0; cp < MAXCP; ++cp) {
      if (cp >= ncp) break;
#pragma unroll
      for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
        for (int dt = 0; dt < (NDP > 0 ? 2 : 1); ++dt) {
          const typename E::frag a = D >= 32 ? TL::load_tr(sX, 32 * cp, 32 * dp + 4 * dt, 8)
                                             : TL::load_tr(sX, 32 * cp, 0, 4);
          acc[dp][dt][0] = E::mma(a, pf[cp], acc[dp][dt][0]);
        }
    }
    if (row_ok) {
      T* dst = (LAST ? (uout ? uout : qhat) : ktil) + row * D;
      if (NDP > 0) {
#pragma unroll
        for (int dp = 0; dp < NACC; ++dp) {
          float o[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] = acc[dp][j >> 2][0][j & 3];
          E::store8(dst + 32 * dp + 8 * G, o);
        }
      } else {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = acc[0][0][0][i];
        E::store4(dst + 4 * G, o);
      }
    }
    if (!LAST && row_ok && G == 0) hent[row] = h2;
  }
  }
}

template <typename T, int D, bool LAST>
__global__ __launch_bounds__(512) void k_rstep(const T* __restrict__ k, const T* __restrict__ v, T* qhat,
                                               T* __restrict__ ktil, float* __restrict__ hent, T* uout,
                                               RGeom p) {
  rstep_body<T, D, LAST>(k, v, qhat, ktil, hent, uout, p, xcd_remap(blockIdx.x, gridDim.x));
}

// Iteration `it` of a run that stops each head on its own: stop_at[bh] is the
// iteration after which head bh stops (0 = not decided).  Two launches per
// iteration: LAST = true gives R V (the last R-step) to the heads that stop
// now (stop_at == it), LAST = false the next L-step's keys and entropies to
// the heads that go on (stop_at == 0); heads that stopped earlier are skipped
// by both.  Each launch has the LDS of its own form and one workgroup per
// key block (a workgroup that looped over several key blocks would wait for
// the stores of one before the loads of the next: measured 20% slower), and
// every workgroup returns at once when no head is left for the launch:
// nstop_upto[i] counts the heads stopped after iteration <= i, so
// nstop_upto[it] - nstop_upto[it - 1] heads stop now and BH - nstop_upto[it]
// go on.
template <typename T, int D, bool LAST>
__global__ __launch_bounds__(512) void k_rstep_adaptive(const T* __restrict__ k, const T* __restrict__ v,
                                                        T* qhat, T* __restrict__ ktil, float* __restrict__ hent,
                                                        const int* __restrict__ stop_at, int it, RGeom p,
                                                        const int* __restrict__ nstop_upto) {
  const int done_before = nstop_upto[it - 1], done_now = nstop_upto[it];
  if (LAST ? done_now == done_before : done_now >= p.BH) return;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int sa = stop_at[item / p.b1];
  if (LAST ? sa != it : sa != 0) return;
  rstep_body<T, D, LAST>(k, v, qhat, LAST ? nullptr : ktil, LAST ? nullptr : hent, nullptr, p, item);
}

}  // namespace monarch
