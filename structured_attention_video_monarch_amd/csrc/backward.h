// Backward kernels of MonarchAttention: the gradient of sum(dy * y) with
// respect to q, k and v, as needed to finetune a video model with the
// attention in place (yunpan.plus MonarchRT article, "Innovation 3:
// finetuning and efficient kernels": the one-iteration form is trained),
// through one or several unrolled iterations, for the square layer and for a
// chunk of query frames against cached keys (query blocks b1r, key blocks b1).
//
// One iteration, R starting uniform (keys of the L-step are the block means
// Kbar, whose entropy term is the same for every block and cancels):
//   L = softmax_c1(s<q_n, Kbar[c1]>), beta = sum_(a1 in g) L,
//   Qh = sum_(a1 in g) L q / beta, R = softmax_c2(s<Qh, k>), U = R V,
//   y_n = sum_c1 L U.
// Reverse (chain rule, in the order the kernels run):
//   kb_du           dU[g,c1,a2] = sum_(a1 in g) L dy
//   kb_rside_a      per key block c1: dR = <dU, v>, dz = R (dR - <R, dR>),
//                   G = s (sum_c2 dz k) / beta, e = <G, Qh>
//   kb_dq           per row n: ghat = sum_c1 L G, delta = <dy,y> + <q,ghat> - sum_c1 L e,
//                   dl = L (<dy,U> + <q,G> - e - delta), dq = ghat + s sum_c1 dl Kbar,
//                   and stores s*dl
//   kb_dkbar        dKbar[c1] = sum_n (s dl)[n,c1] q_n  (partial sums over chunks of n,
//                   then kb_dkbar_reduce)
//   kb_rside_b      per key block c1: dv = sum_(g,a2) R dU,
//                   dk = s sum_(g,a2) dz Qh + dKbar / b2
// Several iterations: the L-step of iteration i > 1 has the keys Kt = R k and
// entropies H of the R-step before; its dl gives dKt and dH (kb_dktil), which
// the R-step kernels of iteration i - 1 take back (their MID forms), and dq,
// dk add up over the iterations in fp32.
// MFMA operand conventions and the slot permutation are those of the forward
// kernels (device_common.h); logits are in log2 units with c = log2(e)/sqrt(d)
// and the log-sum-exps saved by the forward are in the same units.
#pragma once

#include "lside.h"

namespace monarch {

struct BGeom {
  int BH, N, b1, b2, t;
  int b2p;     // b2 rounded up to 32
  float c;     // log2(e) / sqrt(d)
  float s;     // 1 / sqrt(d)
  int nks;     // kb_rside_b: slices of a key block's b2 keys (1 unless b2 > 128)
  int ksw;     // kb_rside_b: keys per slice
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

// The same dot product with x already in registers as the row fragments of a
// contraction over d (lane slots d = 32s + 8G + j: the accumulator's layout
// when D >= 32, so s = dp and j = 4dt + i).
template <typename T, int NACC, int RW>
__device__ inline float dot_acc_frags(const typename Elem<T>::frag (&x)[NACC], const f32x4 (&acc)[NACC][2][RW],
                                      int rt) {
  float r = 0.0f;
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int j = 0; j < 8; ++j) r += Elem<T>::slot(x[dp], j) * acc[dp][j >> 2][rt][j & 3];
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

// ---------------------------------------------------------------- kb_du --
// Column pass: one workgroup owns CB = NW*RW*16 key blocks c1 of tile g in
// column a2; the rows a1 of the tile stream through LDS in steps of 64,
// double-buffered by DMA:  dU[g,c1,a2] = sum_(a1 in g) L[a1,c1] dy_(a1,a2),
// computed as dU^T = dy^T P (the forward's aggregation with dy as values).
// Keys of the L-step: the block means (BCAST) or, after two or more
// iterations, the aggregated keys and entropies (bits) of the R-step before.
template <typename T, int D, int RW, int NW, bool BCAST = true>
__global__ __launch_bounds__(NW * kWave) void kb_du(const T* __restrict__ q, const T* __restrict__ dy,
                                                    const T* __restrict__ kt, const float* __restrict__ h2,
                                                    const float* __restrict__ lse, T* __restrict__ du, LGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int CB = NW * RW * 16;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  // two stages' buffers as distinct LDS objects in a fixed alternation: the
  // prefetch is not waited for before the current stage's reads
  __shared__ __align__(16) T sQ0[kStep * DK];
  __shared__ __align__(16) T sQ1[kStep * DK];
  __shared__ __align__(16) T sY0[kStep * DK];
  __shared__ __align__(16) T sY1[kStep * DK];
  __shared__ __align__(16) float sL0[kStep];
  __shared__ __align__(16) float sL1[kStep];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nrb;
  int rest = logical / p.nrb;
  const int a2 = rest % p.b2;
  rest /= p.b2;
  const int g = rest % p.t;
  const int bh = rest / p.t;
  const int lo = tile_lo(g, p.b1r, p.t), hi = tile_lo(g + 1, p.b1r, p.t);
  const int nrows = hi - lo;
  const int nst = (nrows + kStep - 1) / kStep;

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const long long hoff = static_cast<long long>(bh) * p.N;
  const long long qstride = static_cast<long long>(p.b2) * D;
  const long long gbase = (static_cast<long long>(bh) * p.t + g) * p.b1;  // (bh, g, c1 = 0)

  auto fetch = [&](int st, T* tQ, T* tY, float* tL) {
    const long long n_first = hoff + static_cast<long long>(lo + st * kStep) * p.b2 + a2;
    const int nvalid = nrows - st * kStep;
    Dma::issue(tQ, q + n_first * D, qstride, nvalid);
    Dma::issue(tY, dy + n_first * D, qstride, nvalid);
    if (wave == NW - 1) dma_floats64(tL, lse + n_first, p.b2, nvalid);
  };
  fetch(0, sQ0, sY0, sL0);

  typename E::frag bk[RW][KS];
  float hb[RW];  // entropy bias of the lane's key block
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = cb * CB + (wave * RW + rt) * 16 + l16;
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

  auto stage = [&](int st, const T* cQ, const T* cY, const float* cL, T* nQ, T* nY, float* nL) {
    if (st + 1 < nst) fetch(st + 1, nQ, nY, nL);
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
      const int k0 = 32 * half;
      const int r0 = st * kStep + k0;
      if (r0 >= nrows) break;
      const bool tail = r0 + 32 > nrows;
      typename E::frag a[KS][2];
      load_rows<T, DK, KS>(a, cQ, k0, l16, G);
      float lr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) lr[j] = cL[k0 + 8 * G + j];
      f32x4 S[2][RW];
      logits<T, KS, RW>(S, a, bk);
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, hb[rt] - lr[j]));
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = r0 + 8 * G + j < nrows ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, cY, k0);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 2) {
    stage(st, sQ0, sY0, sL0, sQ1, sY1, sL1);
    if (st + 1 < nst) stage(st + 1, sQ1, sY1, sL1, sQ0, sY0, sL0);
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = cb * CB + (wave * RW + rt) * 16 + l16;
    if (c1 >= p.b1) continue;
    store_rows<T, D, NACC, RW>(du + ((gbase + c1) * p.b2 + a2) * D, acc, rt, 1.0f, G);
  }
}

// ------------------------------------------------------------- kb_du_col --
// Same result as kb_du for tiles of at most kColRows rows (bf16): one
// workgroup owns the whole tile column (bh, g, a2); its q and dy rows and
// log-sum-exps are copied to LDS once, and each wave then takes the key tiles
// wave, wave + NW, ... (RW*16 key blocks each) of all b1 key blocks with no
// further barrier: the column is read once for every key block instead of
// once per CB of them.
template <typename T, int D, int RW, int NW, bool BCAST = true>
__global__ __launch_bounds__(NW * kWave) void kb_du_col(const T* __restrict__ q, const T* __restrict__ dy,
                                                        const T* __restrict__ kt, const float* __restrict__ h2,
                                                        const float* __restrict__ lse, T* __restrict__ du, LGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using Dma = TileDma<T, D, DK, kStep, NW>;
  constexpr int NSTEP = kColRows / kStep;
  __shared__ __align__(16) T sQ[NSTEP][kStep * DK];
  __shared__ __align__(16) T sY[NSTEP][kStep * DK];
  __shared__ __align__(16) float sL[NSTEP][kStep];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int a2 = logical % p.b2;
  const int rest = logical / p.b2;
  const int g = rest % p.t;
  const int bh = rest / p.t;
  const int lo = tile_lo(g, p.b1r, p.t), hi = tile_lo(g + 1, p.b1r, p.t);
  const int nrows = hi - lo;
  const int nst = (nrows + kStep - 1) / kStep;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const long long hoff = static_cast<long long>(bh) * p.N;
  const long long qstride = static_cast<long long>(p.b2) * D;
  const long long gbase = (static_cast<long long>(bh) * p.t + g) * p.b1;  // (bh, g, c1 = 0)

  for (int st = 0; st < nst; ++st) {
    const long long n_first = hoff + static_cast<long long>(lo + st * kStep) * p.b2 + a2;
    const int nvalid = nrows - st * kStep;
    Dma::issue(sQ[st], q + n_first * D, qstride, nvalid);
    Dma::issue(sY[st], dy + n_first * D, qstride, nvalid);
    if (wave == NW - 1) dma_floats64(sL[st], lse + n_first, p.b2, nvalid);
  }
  __syncthreads();

  const int nkt = (p.b1 + RW * 16 - 1) / (RW * 16);
  const int nblk = (nrows + 31) / 32;
  constexpr int kMaxBlk = kColRows / 32;
  // a last block of at most 16 rows takes half the logits and exponentials
  // (as in k_aggregate_col)
  constexpr bool kHalfOk = MONARCH_AGG_HALF && BCAST && sizeof(T) == 2 && D >= 32;
  const bool half_last = kHalfOk && nrows - 32 * (nblk - 1) <= 16;
  const int nfull = half_last ? nblk - 1 : nblk;
  for (int ktile = wave; ktile < nkt; ktile += NW) {
    const int c1base = ktile * RW * 16;
    typename E::frag bk[RW][KS];
    float hb[RW];  // entropy bias of the lane's key block
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      const int c1 = c1base + rt * 16 + l16;
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

#pragma unroll
    for (int blk = 0; blk < kMaxBlk; ++blk) {
      if (blk >= nfull) break;
      const int st = blk / kHalves, k0 = 32 * (blk % kHalves);
      const int r0 = 32 * blk;
      const bool tail = r0 + 32 > nrows;
      typename E::frag a[KS][2];
      load_rows<T, DK, KS>(a, sQ[st], k0, l16, G);
      float lr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) lr[j] = sL[st][k0 + 8 * G + j];
      f32x4 S[2][RW];
      logits<T, KS, RW>(S, a, bk);
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, hb[rt] - lr[j]));
        if (tail) {
          const int lim = nrows - r0 - 8 * G;  // rows of this lane group still in the tile
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = j < lim ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, sY[st], k0);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    if constexpr (kHalfOk) {
      if (half_last) {
        // rows r0 .. r0+15 in natural order: logit slot 4G+i is row 4G+i and
        // lands in contraction slot 8G+i; slots 8G+4..7 get weight 0 (and
        // zero values)
        const int st = nfull / kHalves, k0 = 32 * (nfull % kHalves);
        const int r0 = 32 * nfull;
        typename E::frag a[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = Tile<T, DK>::load8(sQ[st], k0 + l16, s * 32 + 8 * G);
        float lr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lr[i] = sL[st][k0 + 4 * G + i];
        const int lim = nrows - r0 - 4 * G;
        typename E::frag pf[RW];
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) {
          f32x4 S0 = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < KS; ++s) S0 = E::mma(a[s], bk[rt][s], S0);
          float w[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = fast_exp2(__builtin_fmaf(S0[i], p.c, hb[rt] - lr[i]));
            w[i] = i < lim ? x : 0.0f;
            w[4 + i] = 0.0f;
          }
          pf[rt] = E::pack(w);
        }
        typename E::frag vv[NACC][2];
#pragma unroll
        for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) vv[dp][dt] = Tile<T, DK>::load_tr_half(sY[st], k0, 32 * dp + 4 * dt, 8);
        weighted_sum<T, D, NACC, RW>(acc, vv, pf);
      }
    }

#pragma unroll
    for (int rt = 0; rt < RW; ++rt) {
      const int c1 = c1base + rt * 16 + l16;
      if (c1 >= p.b1) continue;
      store_rows<T, D, NACC, RW>(du + ((gbase + c1) * p.b2 + a2) * D, acc, rt, 1.0f, G);
    }
  }
}

// ------------------------------------------------------------- kb_rside_a --
// Key-block pass, part 1 (as the forward R-step): one workgroup per (bh, c1);
// K and V of the block are copied to LDS once, and the waves share out the
// tasks (tile g, 16 rows a2) of the block, each task's rows of the
// aggregated queries Qh and of dU loaded by its wave (no barrier inside the
// loop).  With ceil(b2/16) waves a wave keeps one row tile through all
// tiles g; with four waves (bf16, at most 168 registers) three workgroups
// share a CU, twelve waves where one workgroup of five waves did before.
// Per (g, c1, a2), from the transposed logits (rows c2, columns a2):
//   R = softmax_c2(s<Qh, k>), dR = <dU, v>, rho = <R, dR>, dz = R (dR - rho),
//   G = s (K^T dz) / beta, e = <G, Qh>; stored: G, e and the row statistics
//   (log-sum-exp of the logits in log2 units, and rho) for part 2.
// MID (an R-step before the last, whose R feeds the next L-step as the keys
// Kt = R k and entropies H = -sum R ln R): the cotangents are dKt and dH
// (passed in du and dh), so dR = <dKt, k> - dH (ln R + 1); the constant
// drops out of dz because R sums to 1, and keys past b2 (R = 0) get dR = 0.
template <typename T, int D>
inline size_t rside_bwd_lds_bytes(int b2p) {
  const int DK = D < 32 ? 32 : D;
  return sizeof(T) * static_cast<size_t>(b2p) * DK * 2;
}

// Global -> LDS DMA of `rows` rows of a contiguous [rows][D] block into a
// swizzled tile (rows >= nvalid repeat row nvalid-1); nw waves take part.
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

// waves per kb_rside_a workgroup when a block has at least 2 tasks per wave
#ifndef MONARCH_BRA_NW
#define MONARCH_BRA_NW 4
#endif
// minimum waves per SIMD the register allocator must allow
#ifndef MONARCH_BRA_MINW
#define MONARCH_BRA_MINW 1
#endif
#ifndef MONARCH_BRB_MINW
#define MONARCH_BRB_MINW 1
#endif

template <typename T, int D, int NCP, bool MID = false>
__global__ __launch_bounds__(512, MONARCH_BRA_MINW) void kb_rside_a(const T* __restrict__ k, const T* __restrict__ v,
                                                  const T* __restrict__ qhat, const T* __restrict__ du,
                                                  const float* __restrict__ dh,
                                                  const float* __restrict__ beta, T* __restrict__ gq,
                                                  float* __restrict__ ev, float* __restrict__ lser,
                                                  float* __restrict__ rho, BGeom p) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using TL = Tile<T, DK>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int b2p = p.b2p;
  T* sK = reinterpret_cast<T*>(smem_raw);
  T* sV = MID ? sK : sK + b2p * DK;  // MID: the cotangent pairs with k

  const int item = xcd_remap(blockIdx.x, gridDim.x);  // bh*b1 + c1
  const int c1 = item % p.b1;
  const int bh = item / p.b1;
  const long long blk = static_cast<long long>(item) * p.b2;  // first key row of block c1
  const int nw = blockDim.x / kWave;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  // tasks: (tile g, 16 rows a2) pairs, task = g * ntr + row tile; wave w
  // takes tasks w, w + nw, ...
  const int ntr = (p.b2 + 15) / 16;
  const int ntask = p.t * ntr;

  dma_block<T, D, DK>(sK, k + blk * D, b2p, p.b2, nw);
  if (!MID) dma_block<T, D, DK>(sV, v + blk * D, b2p, p.b2, nw);

  // a task's operands: its rows of Qh and dU (B fragments), beta and dH
  struct Ops {
    typename E::frag q[KS], d[KS];
    float bt, dhv;
  };
  auto row_of = [&](int task, bool& row_ok) {
    const int g = task / ntr;
    const int a2 = (task - g * ntr) * 16 + l16;
    row_ok = a2 < p.b2;
    return ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2 + a2;
  };
  auto load_ops = [&](int task, Ops& o) {
    bool row_ok;
    const long long row = row_of(task, row_ok);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = s * 32 + 8 * G;
      const bool ok = row_ok && col < D;
      o.q[s] = ok ? E::load(qhat + row * D + col) : E::zero();
      o.d[s] = ok ? E::load(du + row * D + col) : E::zero();
    }
    o.bt = row_ok ? beta[row] : 0.0f;
    // MID: dH of this row in nats per log2 unit of the logit
    o.dhv = MID && row_ok ? dh[row] * kLn2 : 0.0f;
  };
  auto run_task = [&](int task, const Ops& o) {
    // K and V never change in LDS during the loop: without this fence the
    // compiler hoists every fragment read of them out of the task loop
    // (about 190 registers) and spills
    asm volatile("" ::: "memory");
    bool row_ok;
    const long long row = row_of(task, row_ok);
    f32x4 S[NCP][2], DR[NCP][2];
#pragma unroll
    for (int cp = 0; cp < NCP; ++cp) {
      S[cp][0] = S[cp][1] = DR[cp][0] = DR[cp][1] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int r = 32 * cp + perm_row(ct, l16);
          S[cp][ct] = E::mma(TL::load8(sK, r, 32 * s + 8 * G), o.q[s], S[cp][ct]);
          DR[cp][ct] = E::mma(TL::load8(sV, r, 32 * s + 8 * G), o.d[s], DR[cp][ct]);
        }
    }
    // softmax over c2 = 32cp + 8G + j for column a2 (keys past b2 masked)
    float x[NCP][8];
    float mx = -1e30f;
#pragma unroll
    for (int cp = 0; cp < NCP; ++cp)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c2 = 32 * cp + 8 * G + j;
        x[cp][j] = c2 < p.b2 ? S[cp][j >> 2][j & 3] * p.c : kNegInf;
        mx = fmaxf(mx, x[cp][j]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.0f;
#pragma unroll
    for (int cp = 0; cp < NCP; ++cp)
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += fast_exp2(x[cp][j] - mx);
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    const float lse2 = mx + log2f(sum);
    // MID: dH of this row in nats per log2 unit of the logit
    const float dhl = o.dhv;
    float rh = 0.0f;
#pragma unroll
    for (int cp = 0; cp < NCP; ++cp)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (MID) {
          const bool valid = 32 * cp + 8 * G + j < p.b2;
          DR[cp][j >> 2][j & 3] = valid ? DR[cp][j >> 2][j & 3] - dhl * (x[cp][j] - lse2) : 0.0f;
        }
        x[cp][j] = fast_exp2(x[cp][j] - lse2);  // now R
        rh += x[cp][j] * DR[cp][j >> 2][j & 3];
      }
    rh += __shfl_xor(rh, 16);
    rh += __shfl_xor(rh, 32);
    // dQh^T = K^T dz^T: rows d, columns a2
    f32x4 acc[NACC][2][1];
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) acc[dp][0][0] = acc[dp][1][0] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int cp = 0; cp < NCP; ++cp) {
      float z[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) z[j] = x[cp][j] * (DR[cp][j >> 2][j & 3] - rh);
      const typename E::frag zf = E::pack(z);
#pragma unroll
      for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
        for (int dt = 0; dt < (NDP > 0 ? 2 : 1); ++dt)
          acc[dp][dt][0] = E::mma(load_vals_tr<T, D, DK>(sK, 32 * cp, dp, dt), zf, acc[dp][dt][0]);
    }
    const float bt = o.bt;
    const float sc = bt > 0.0f ? p.s / bt : 0.0f;
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) {
      acc[dp][0][0] *= sc;
      acc[dp][1][0] *= sc;
    }
    // e = <G, Qh> with the rounded Qh the forward used (held in o.q: its
    // lane slots are the accumulator's d positions)
    float e;
    if constexpr (D >= 32)
      e = dot_acc_frags<T, NACC, 1>(o.q, acc, 0);
    else
      e = dot_acc_row<T, D, NACC, 1>(qhat + (row_ok ? row : 0) * D, acc, 0, G);
    e += __shfl_xor(e, 16);
    e += __shfl_xor(e, 32);
    if (row_ok) {
      store_rows<T, D, NACC, 1>(gq + row * D, acc, 0, 1.0f, G);
      if (G == 0) {
        ev[row] = e;
        lser[row] = lse2;
        rho[row] = rh;
      }
    }
  };

  Ops o;
  if (wave < ntask) load_ops(wave, o);
  __syncthreads();
  for (int task = wave; task < ntask; task += nw) {
    if (task != wave) load_ops(task, o);
    run_task(task, o);
  }
}

// ------------------------------------------------------------- kb_rside_b --
// Key-block pass, part 2: one workgroup per (bh, c1), each wave owning
// RW*16 keys c2 (K and V rows as B operands).  The rows (g, a2) of all tiles
// stream through LDS as one sequence of t*b2 rows in blocks of 32 (a block
// may straddle two tiles: rows are gathered by address), BPS blocks per
// double-buffered DMA stage.  R and dz are recomputed from the stored row
// statistics with the rows as the contraction index, and
//   dv[c1,c2] = sum_(g,a2) R dU,
//   dk[c1,c2] = s sum_(g,a2) dz Qh + dKbar[c1] / b2   (dKbar already reduced).
// With several iterations dk collects one term per R-step in the fp32
// dk_acc, by MODE:
//   kRbSingle  one iteration: dv and dk as above;
//   kRbLast    last R-step: dv, and dk_acc = s sum dz Qh;
//   kRbMid     an earlier R-step (du holds dKt, dh holds dH, dR as in
//              kb_rside_a): dk_acc += s sum dz Qh + sum R dKt;
//   kRbFirst   the first R-step (also MID): dk = dk_acc + s sum dz Qh +
//              sum R dKt + dKbar / b2.
constexpr int kRbSingle = 0, kRbLast = 1, kRbMid = 2, kRbFirst = 3;
#ifndef MONARCH_BRB_BPS
#define MONARCH_BRB_BPS 4
#endif
#ifndef MONARCH_BRB_RW
#define MONARCH_BRB_RW 1
#endif

// Row j0 + r (0 <= r < 64; past `total`, the last row) of the sequence of
// t*b2 rows (g, a2) of one key block: rbase + (j / b2) * tstride + j % b2.
// j0 is the same for the whole wave, so its split into (g, a2) is scalar
// work; the lane's offset r then wraps past b2 at most twice when b2 >= 32
// (a division per lane only for shorter key blocks).
// Row of the sequence position j0 + r relative to rbase: g * tstride + a,
// below t*N < 2^31 (the shape envelope).
__device__ inline unsigned seq_row_rel(long long tstride, int j0, int r, int total, int b2) {
  if (j0 + r >= total) r = total - 1 - j0;
  const int g0 = j0 / b2;
  int a = j0 - g0 * b2 + r, g = g0;
  if (b2 >= 32) {
    if (a >= b2) { a -= b2; ++g; }
    if (a >= b2) { a -= b2; ++g; }
  } else {
    g += a / b2;
    a %= b2;
  }
  return static_cast<unsigned>(g) * static_cast<unsigned>(tstride) + static_cast<unsigned>(a);
}

// Global -> LDS DMA of 32 rows j0 .. j0+31 of the sequence of t*b2 rows
// (g, a2) of one key block: row j lives at rbase + (j / b2) * tstride + j % b2
// (rows past `total` repeat the last row).
template <typename T, int D, int DK>
__device__ inline void dma_rows32(T* tile, const T* src, long long rbase, int j0, int total, int b2,
                                  long long tstride, int nw) {
  constexpr int V = Elem<T>::kVec;
  constexpr int ROWB = DK * static_cast<int>(sizeof(T));
  constexpr int NINS = 32 * ROWB / 1024;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave)), lane = lane_id();
  for (int ci = wave; ci < NINS; ci += nw) {
    const int byte = ci * 1024 + 16 * lane;
    const int r = byte / ROWB;
    const int c = ((byte % ROWB) / 16) ^ Tile<T, DK>::swz(r);
    int col = c * V;
    if (col >= D) col -= D;
    const unsigned rel = seq_row_rel(tstride, j0, r, total, b2);
    // bf16: the byte offset from the block's first row fits 32 bits (t*N*d <
    // 2^31 elements), so it is a lane offset on a wave-uniform base
    const void* a = sizeof(T) == 2
        ? static_cast<const void*>(reinterpret_cast<const char*>(src + rbase * D) + (rel * D + col) * 2u)
        : static_cast<const void*>(src + (rbase + rel) * D + col);
    __builtin_amdgcn_global_load_lds(a,
                                     (__attribute__((address_space(3))) void*)(tile + ci * (1024 / static_cast<int>(sizeof(T)))),
                                     16, 0, 0);
  }
}

// The same for one float per row (64 lanes, rows j0 .. j0+63).
__device__ inline void dma_rowstat(float* dst, const float* src, long long rbase, int j0, int total, int b2,
                                   long long tstride) {
  const unsigned rel = seq_row_rel(tstride, j0, lane_id(), total, b2);
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(reinterpret_cast<const char*>(src + rbase) + rel * 4u),
                                   (__attribute__((address_space(3))) void*)(dst), 4, 0, 0);
}

template <typename T, int D, int MODE = kRbSingle, int RWK = MONARCH_BRB_RW>
__global__ __launch_bounds__(RWK == 1 || RWK != MONARCH_BRB_RW ? 512 : 256, MONARCH_BRB_MINW) void kb_rside_b(const T* __restrict__ k, const T* __restrict__ v,
                                                  const T* __restrict__ qhat, const T* __restrict__ du,
                                                  const float* __restrict__ lser, const float* __restrict__ rho,
                                                  const float* __restrict__ dh,
                                                  const float* __restrict__ dkbar, T* __restrict__ dk,
                                                  float* __restrict__ dk_acc, T* __restrict__ dv, BGeom p) {
  constexpr bool MID = MODE == kRbMid || MODE == kRbFirst;
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  // 32-row blocks per pipeline stage (f32 tiles are twice as large: one)
  constexpr int BPS = sizeof(T) == 2 ? MONARCH_BRB_BPS : 1;
  constexpr int RW = RWK;
  __shared__ __align__(16) T sQ[2][BPS][32 * DK];
  __shared__ __align__(16) T sU[2][BPS][32 * DK];
  __shared__ __align__(16) float sLR[2][BPS][64];
  __shared__ __align__(16) float sRh[2][BPS][64];
  __shared__ __align__(16) float sDh[MID ? 2 : 1][MID ? BPS : 1][64];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);  // (bh*b1 + c1)*nks + slice
  const int slice = logical % p.nks;
  const int item = logical / p.nks;  // bh*b1 + c1
  const int c1 = item % p.b1;
  const int bh = item / p.b1;
  const long long blk = static_cast<long long>(item) * p.b2;
  const int kofs = slice * p.ksw;  // the slice's first key c2
  const int nw = blockDim.x / kWave;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const int total = p.t * p.b2;               // rows (g, a2) of all tiles, in order
  const int nblk = (total + 31) / 32;
  const int nst = (nblk + BPS - 1) / BPS;
  const long long rbase = (static_cast<long long>(bh) * p.t * p.b1 + c1) * p.b2;  // row (g = 0, c1, a2 = 0)
  const long long tstride = static_cast<long long>(p.b1) * p.b2;                  // rows between tiles

  auto fetch = [&](int st, int buf) {
#pragma unroll
    for (int j = 0; j < BPS; ++j) {
      const int b = st * BPS + j;
      if (b >= nblk) break;
      const int j0 = 32 * b;
      dma_rows32<T, D, DK>(sQ[buf][j], qhat, rbase, j0, total, p.b2, tstride, nw);
      dma_rows32<T, D, DK>(sU[buf][j], du, rbase, j0, total, p.b2, tstride, nw);
      if (wave == 0) dma_rowstat(sLR[buf][j], lser, rbase, j0, total, p.b2, tstride);
      if (wave == nw - 1) dma_rowstat(sRh[buf][j], rho, rbase, j0, total, p.b2, tstride);
      if (MID && wave == 1 % nw) dma_rowstat(sDh[MID ? buf : 0][MID ? j : 0], dh, rbase, j0, total, p.b2, tstride);
    }
  };
  fetch(0, 0);

  typename E::frag bk2[RW][KS], bv2[RW][KS];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c2 = kofs + (wave * RW + rt) * 16 + l16;
    const int c2c = c2 < p.b2 ? c2 : p.b2 - 1;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int col = 32 * s + 8 * G;
      bk2[rt][s] = col < D ? E::load(k + (blk + c2c) * D + col) : E::zero();
      bv2[rt][s] = (!MID && col < D) ? E::load(v + (blk + c2c) * D + col) : E::zero();
    }
  }
  f32x4 accv[NACC][2][RW], acck[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) accv[dp][dt][rt] = acck[dp][dt][rt] = f32x4{0, 0, 0, 0};
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) fetch(st + 1, cur ^ 1);
#pragma unroll
    for (int j = 0; j < BPS; ++j) {
      const int b = st * BPS + j;
      if (b >= nblk) break;
      const int j0 = 32 * b;
      const T* tq = sQ[cur][j];
      const T* tu = sU[cur][j];
      typename E::frag a[KS][2];
      f32x4 Z[2][RW], DR[2][RW];
      load_rows<T, DK, KS>(a, tq, 0, l16, G);
      logits<T, KS, RW>(Z, a, bk2);
      load_rows<T, DK, KS>(a, tu, 0, l16, G);
      if (MID)
        logits<T, KS, RW>(DR, a, bk2);  // <dKt, k>
      else
        logits<T, KS, RW>(DR, a, bv2);  // <dU, v>
      typename E::frag rf[RW], zf[RW];
      const bool tail = j0 + 32 > total;  // rows past the sequence repeat the last row: weight 0
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float r[8], z[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float xl = Z[jj >> 2][rt][jj & 3] * p.c - sLR[cur][j][8 * G + jj];  // log2 R
          const float rr = fast_exp2(xl);
          float dr = DR[jj >> 2][rt][jj & 3];
          if (MID) dr -= sDh[MID ? cur : 0][MID ? j : 0][8 * G + jj] * kLn2 * xl;
          r[jj] = rr;
          z[jj] = rr * (dr - sRh[cur][j][8 * G + jj]);
        }
        if (tail) {
          const int lim = total - j0 - 8 * G;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            r[jj] = jj < lim ? r[jj] : 0.0f;
            z[jj] = jj < lim ? z[jj] : 0.0f;
          }
        }
        rf[rt] = E::pack(r);
        zf[rt] = E::pack(z);
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, tu, 0);
      weighted_sum<T, D, NACC, RW>(accv, vv, rf);
      load_cols<T, D, DK, NACC>(vv, tq, 0);
      weighted_sum<T, D, NACC, RW>(acck, vv, zf);
    }
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c2 = kofs + (wave * RW + rt) * 16 + l16;
    if (c2 >= p.b2) continue;
    const long long orow = (blk + c2) * D;
    if (!MID) store_rows<T, D, NACC, RW>(dv + orow, accv, rt, 1.0f, G);
    // this R-step's key gradient over the lane's d positions (32dp + 8G + j,
    // or 4G + j when D == 16), combined as MODE says; dkbar holds the
    // block-mean gradient already divided by b2
    const float* mk = dkbar + static_cast<long long>(item) * D;
    constexpr int NJ = D >= 32 ? 8 : 4;
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) {
      const int d0 = D >= 32 ? 32 * dp + 8 * G : 4 * G;
      float o[8];
#pragma unroll
      for (int jd = 0; jd < NJ; ++jd) {
        o[jd] = p.s * acck[dp][jd >> 2][rt][jd & 3];
        if (MID) o[jd] += accv[dp][jd >> 2][rt][jd & 3];
        if (MODE == kRbSingle || MODE == kRbFirst) o[jd] += mk[d0 + jd];
        if (MODE == kRbMid || MODE == kRbFirst) o[jd] += dk_acc[orow + d0 + jd];
      }
      if (MODE == kRbSingle || MODE == kRbFirst) {
        if (D >= 32)
          E::store8(dk + orow + d0, o);
        else
          E::store4(dk + orow + d0, o);
      } else {
#pragma unroll
        for (int jd = 0; jd < NJ; ++jd) dk_acc[orow + d0 + jd] = o[jd];
      }
    }
  }
}

// ------------------------------------------------------------------ kb_dq --
// Row pass (as k_apply): one workgroup owns RB = NW*RW*16 rows a1 of tile g
// in column a2.  Pass 1 over c1: ghat = sum L G and eps = sum L e (a product
// with e in every row of the A operand), then delta = <dy,y> + <q,ghat> - eps.
// Pass 2 over c1: dl = L (<dy,U> + <q,G> - e - delta) and
// dq = ghat + s sum_c1 dl Kt; s*dl (as rounded for the product) is also
// stored, [n][c1] with row stride ldl, for the key gradient.
// The L-step's keys Kt are the block means (BCAST, first iteration) or the
// aggregated keys and entropies of the R-step before.  Without HAS_DY (an
// earlier iteration, whose L feeds only the aggregation) the dy, y and U
// terms are absent.  Over several iterations dq collects one term per L-step
// in the fp32 dq_acc, by DQM:
constexpr int kDqStore = 0;   // one iteration: dq = this term
constexpr int kDqInit = 1;    // last L-step: dq_acc = this term
constexpr int kDqAdd = 2;     // dq_acc += this term
constexpr int kDqFinish = 3;  // first L-step: dq = dq_acc + this term
template <typename T, int D, int RW, int NW, bool BCAST = true, bool HAS_DY = true, int DQM = kDqStore,
          int STEP = kStep>
__global__ __launch_bounds__(NW * kWave) void kb_dq(const T* __restrict__ q, const T* __restrict__ dy,
                                                    const T* __restrict__ y, const T* __restrict__ kt,
                                                    const float* __restrict__ h2,
                                                    const float* __restrict__ lse, const T* __restrict__ u,
                                                    const T* __restrict__ gq, const float* __restrict__ ev,
                                                    T* __restrict__ dq,
                                                    float* __restrict__ dq_acc,
                                                    T* __restrict__ dlout, int ldl, LGeom p, float sc,
                                                    float kscale = 1.0f) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int KS = DK / 32;
  constexpr int RB = NW * RW * 16;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using Dma = TileDma<T, D, DK, STEP, NW>;
  constexpr int HALVES = STEP / 32;
  // double-buffered for bf16; f32 tiles are twice as large: one buffer
  constexpr int NB = sizeof(T) == 2 ? 2 : 1;
  // the two stages' buffers are distinct LDS objects in a fixed alternation
  // (the prefetch is not waited for before the current stage's reads); with
  // one buffer the second set is the first
  constexpr int TB = STEP * DK;
  __shared__ __align__(16) T sK0[TB];
  __shared__ __align__(16) T sK1[NB == 2 ? TB : 8];
  __shared__ __align__(16) T sU0[HAS_DY ? TB : 8];
  __shared__ __align__(16) T sU1[HAS_DY && NB == 2 ? TB : 8];
  __shared__ __align__(16) T sG0[TB];
  __shared__ __align__(16) T sG1[NB == 2 ? TB : 8];
  __shared__ __align__(16) float sE0[64];  // 64: one float per lane of the DMA
  __shared__ __align__(16) float sE1[64];
  __shared__ __align__(16) float sH0[64];
  __shared__ __align__(16) float sH1[64];
  struct Stage {
    T* K;
    T* U;
    T* G;
    float* E;
    float* H;
  };
  const Stage B0{sK0, sU0, sG0, sE0, sH0};
  const Stage B1 = NB == 2 ? Stage{sK1, sU1, sG1, sE1, BCAST ? sH0 : sH1} : B0;

  ColItem it(p, RB);
  if (it.nrows <= 0) return;
  const int bh = it.bh, g = it.g, a2 = it.a2;
  const long long hoff = static_cast<long long>(bh) * p.N;
  const long long n0 = static_cast<long long>(it.a1_0) * p.b2 + a2;
  const long long nstride = p.b2;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const KeySrc<T, D, BCAST> ks(kt, h2, p, bh, g, a2);
  const long long cbase = (static_cast<long long>(bh) * p.t + g) * p.b1 * p.b2 + a2;  // (bh, g, c1 = 0, a2)
  const long long ustride = static_cast<long long>(p.b2) * D;

  const int nst = (p.b1 + STEP - 1) / STEP;
  auto fetch = [&](int st, const Stage& t, bool with_u) {
    const int c1 = st * STEP;
    Dma::issue(t.K, ks.k + c1 * ks.kstride, ks.kstride, p.b1 - c1);
    Dma::issue(t.G, gq + (cbase + static_cast<long long>(c1) * p.b2) * D, ustride, p.b1 - c1);
    if (HAS_DY && with_u) Dma::issue(t.U, u + (cbase + static_cast<long long>(c1) * p.b2) * D, ustride, p.b1 - c1);
    if (wave == NW - 1) dma_floats64(t.E, ev + cbase + static_cast<long long>(c1) * p.b2, p.b2, p.b1 - c1);
    if (!BCAST && wave == 0) dma_floats64(t.H, ks.h + static_cast<long long>(c1) * ks.hstride, ks.hstride, p.b1 - c1);
  };
  fetch(0, B0, false);

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

  // ---------------- pass 1: ghat and eps
  auto stage1 = [&](int st, const Stage& c, const Stage& n) {
    if (NB == 2 && st + 1 < nst) fetch(st + 1, n, false);
#pragma unroll
    for (int half = 0; half < HALVES; ++half) {
      const int k0 = 32 * half;
      const int c1_0 = st * STEP + k0;
      if (c1_0 >= p.b1) break;
      const bool tail = c1_0 + 32 > p.b1;
      typename E::frag a[KS][2];
      load_rows<T, DK, KS>(a, c.K, k0, l16, G);
      f32x4 S[2][RW];
      logits<T, KS, RW>(S, a, bq);
      float e8[8], hb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e8[j] = c.E[k0 + 8 * G + j];
        hb[j] = BCAST ? 0.0f : c.H[k0 + 8 * G + j];
      }
      const typename E::frag ef = E::pack(e8);
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, nl[rt] + hb[j]));
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = c1_0 + 8 * G + j < p.b1 ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
        acce[rt] = E::mma(ef, pf[rt], acce[rt]);
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, c.G, k0);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    __syncthreads();
    if (NB == 1 && st + 1 < nst) {
      fetch(st + 1, n, false);
      __syncthreads();
    }
  };
  for (int st = 0; st < nst; st += 2) {
    stage1(st, B0, B1);
    if (st + 1 < nst) stage1(st + 1, B1, B0);
  }
  fetch(0, B0, true);

  // delta = <dy, y> + <q, ghat> - eps (every lane group holds a quarter of d)
  float dlt[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    const bool ok = r < it.nrows;
    const long long row = hoff + n0 + (ok ? r : 0) * nstride;
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
  __syncthreads();

  // keys stored pre-scaled (c Kbar, kscale = c): the products of pass 2 with
  // them are c times the dq term, so ghat is scaled to match here and the
  // sum is divided by c at the end
  if (kscale != 1.0f) {
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        acc[dp][0][rt] *= kscale;
        acc[dp][1][rt] *= kscale;
      }
  }

  // ---------------- pass 2: dl and dq
  float nls[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) nls[rt] = nl[rt] + log2f(sc);
  auto stage2 = [&](int st, const Stage& c, const Stage& n) {
    if (NB == 2 && st + 1 < nst) fetch(st + 1, n, true);
#pragma unroll
    for (int half = 0; half < HALVES; ++half) {
      const int k0 = 32 * half;
      const int c1_0 = st * STEP + k0;
      if (c1_0 >= p.b1) break;
      const bool tail = c1_0 + 32 > p.b1;
      typename E::frag a[KS][2];
      f32x4 S[2][RW], X[2][RW];
      float e8[8], hb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e8[j] = c.E[k0 + 8 * G + j];
        hb[j] = BCAST ? 0.0f : c.H[k0 + 8 * G + j];
      }
      // X = dL - delta accumulates onto -(e + delta): the products start
      // from it, so no subtraction is left per weight
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        X[0][rt] = f32x4{-(e8[0] + dlt[rt]), -(e8[1] + dlt[rt]), -(e8[2] + dlt[rt]), -(e8[3] + dlt[rt])};
        X[1][rt] = f32x4{-(e8[4] + dlt[rt]), -(e8[5] + dlt[rt]), -(e8[6] + dlt[rt]), -(e8[7] + dlt[rt])};
      }
      load_rows<T, DK, KS>(a, c.K, k0, l16, G);
      logits<T, KS, RW>(S, a, bq);
      if (HAS_DY) {
        load_rows<T, DK, KS>(a, c.U, k0, l16, G);
        products<T, KS, RW>(X, a, bdy);  // + <U, dy>
      }
      load_rows<T, DK, KS>(a, c.G, k0, l16, G);
      products<T, KS, RW>(X, a, bq);  // + <G, q>
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        float w[8];
        // s * L: the scale s = 2^lsc rides in the exponent
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[j] = fast_exp2(__builtin_fmaf(S[j >> 2][rt][j & 3], p.c, nls[rt] + hb[j])) * X[j >> 2][rt][j & 3];
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = c1_0 + 8 * G + j < p.b1 ? w[j] : 0.0f;
        }
        pf[rt] = E::pack(w);
        // s*dl of row n, keys c1_0 + 8G .. +7, for the key gradient
        const int r = (wave * RW + rt) * 16 + l16;
        if (r < it.nrows) {
          T* dst = dlout + (hoff + n0 + r * nstride) * ldl + c1_0 + 8 * G;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint4*>(dst) = __builtin_bit_cast(uint4, pf[rt]);
          } else {
            E::store8(dst, w);
          }
        }
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, c.K, k0);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    __syncthreads();
    if (NB == 1 && st + 1 < nst) {
      fetch(st + 1, n, true);
      __syncthreads();
    }
  };
  for (int st = 0; st < nst; st += 2) {
    stage2(st, B0, B1);
    if (st + 1 < nst) stage2(st + 1, B1, B0);
  }
  if (kscale != 1.0f) {
    const float ik = 1.0f / kscale;
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        acc[dp][0][rt] *= ik;
        acc[dp][1][rt] *= ik;
      }
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int r = (wave * RW + rt) * 16 + l16;
    if (r >= it.nrows) continue;
    const long long row = hoff + n0 + r * nstride;
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

// ------------------------------------------------------------- kb_dktil --
// Key-side gradient of an L-step whose keys are the aggregated keys Kt and
// entropies H of the R-step before (second and later iterations): the logit
// s<q_n, Kt[g,c1,a2]> + H[g,c1,a2] of row n = (a1, a2), a1 in tile g, gives
//   dKt[g,c1,a2] = sum_(a1 in g) (s dl)[n,c1] q_n,
//   dH[g,c1,a2]  = sum_(a1 in g) dl[n,c1].
// kb_du's column pass with the stored s*dl as the weights (transposed LDS
// reads of its [rows][keys] block, as in kb_dkbar) instead of L; dH is a
// product with an all-ones A operand, divided by s.
template <typename T, int D, int RW, int NW>
__global__ __launch_bounds__(NW * kWave) void kb_dktil(const T* __restrict__ q, const T* __restrict__ dl, int ldl,
                                                       T* __restrict__ dkt, float* __restrict__ dh, LGeom p,
                                                       float inv_s) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int CB = NW * RW * 16;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using DmaQ = TileDma<T, D, DK, kStep, NW>;
  using DmaL = TileDma<T, CB, CB, kStep, NW>;
  // two stages' buffers as distinct LDS objects in a fixed alternation
  __shared__ __align__(16) T sQ0[kStep * DK];
  __shared__ __align__(16) T sQ1[kStep * DK];
  __shared__ __align__(16) T sL0[kStep * CB];
  __shared__ __align__(16) T sL1[kStep * CB];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = logical % p.nrb;
  int rest = logical / p.nrb;
  const int a2 = rest % p.b2;
  rest /= p.b2;
  const int g = rest % p.t;
  const int bh = rest / p.t;
  const int lo = tile_lo(g, p.b1r, p.t), hi = tile_lo(g + 1, p.b1r, p.t);
  const int nrows = hi - lo;
  const int nst = (nrows + kStep - 1) / kStep;

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  const long long hoff = static_cast<long long>(bh) * p.N;
  const long long qstride = static_cast<long long>(p.b2) * D;
  const long long lstride = static_cast<long long>(p.b2) * ldl;
  const long long gbase = (static_cast<long long>(bh) * p.t + g) * p.b1;  // (bh, g, c1 = 0)

  auto fetch = [&](int st, T* tQ, T* tL) {
    const long long n_first = hoff + static_cast<long long>(lo + st * kStep) * p.b2 + a2;
    const int nvalid = nrows - st * kStep;
    DmaQ::issue(tQ, q + n_first * D, qstride, nvalid);
    DmaL::issue(tL, dl + n_first * ldl + cb * CB, lstride, nvalid);
  };
  fetch(0, sQ0, sL0);

  float one8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) one8[j] = 1.0f;
  const typename E::frag ones = E::pack(one8);
  f32x4 acc[NACC][2][RW];
  f32x4 acch[RW];
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    acch[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int dp = 0; dp < NACC; ++dp) acc[dp][0][rt] = acc[dp][1][rt] = f32x4{0, 0, 0, 0};
  }
  __syncthreads();

  auto stage = [&](int st, const T* cQ, const T* cL, T* nQ, T* nL) {
    if (st + 1 < nst) fetch(st + 1, nQ, nL);
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
      const int k0 = 32 * half;
      const int r0 = st * kStep + k0;
      if (r0 >= nrows) break;
      const bool tail = r0 + 32 > nrows;
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        pf[rt] = Tile<T, CB>::load_tr(cL, k0, (wave * RW + rt) * 16, 4);
        if (tail) {
          // rows past the tile repeat its last row: zero their slots
          float w[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = r0 + 8 * G + j < nrows ? E::slot(pf[rt], j) : 0.0f;
          pf[rt] = E::pack(w);
        }
        acch[rt] = E::mma(ones, pf[rt], acch[rt]);
      }
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, cQ, k0);
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
    }
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 2) {
    stage(st, sQ0, sL0, sQ1, sL1);
    if (st + 1 < nst) stage(st + 1, sQ1, sL1, sQ0, sL0);
  }

#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = cb * CB + (wave * RW + rt) * 16 + l16;
    if (c1 >= p.b1) continue;
    const long long col = (gbase + c1) * p.b2 + a2;
    store_rows<T, D, NACC, RW>(dkt + col * D, acc, rt, 1.0f, G);
    if (G == 0) dh[col] = acch[rt][0] * inv_s;
  }
}

// -------------------------------------------------------------- kb_dkbar --
// dKbar[c1] = s sum_n dl[n,c1] q_n over all tokens n of a head: a plain
// product of the stored s*dl [N x ldl] and q [N x d], split over chunks of n
// (partial sums part[split][c1][d], reduced by kb_dkbar_reduce).  One workgroup:
// (bh, block of CB = NW*RW*16 keys c1, chunk of n); 32 rows n per step,
// double-buffered by DMA; per wave RW key tiles times all of d, computed as
// dKbar^T = q^T dl (both operands by transposing LDS reads).
constexpr int kGemmStep = 32;

template <typename T, int D, int RW, int NW>
__global__ __launch_bounds__(NW * kWave) void kb_dkbar(const T* __restrict__ q, const T* __restrict__ dl, int ldl,
                                                       float* __restrict__ part, int BH, int N, int b1, int ncb,
                                                       int nsplit, int chunk) {
  using E = Elem<T>;
  constexpr int DK = D < 32 ? 32 : D;
  constexpr int CB = NW * RW * 16;
  constexpr int NDP = D / 32;
  constexpr int NACC = NDP > 0 ? NDP : 1;
  using DmaQ = TileDma<T, D, DK, kGemmStep, NW>;
  using DmaL = TileDma<T, CB, CB, kGemmStep, NW>;
  // two stages' buffers as distinct LDS objects in a fixed alternation
  __shared__ __align__(16) T sQ0[kGemmStep * DK];
  __shared__ __align__(16) T sQ1[kGemmStep * DK];
  __shared__ __align__(16) T sL0[kGemmStep * CB];
  __shared__ __align__(16) T sL1[kGemmStep * CB];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int split = logical % nsplit;
  int rest = logical / nsplit;
  const int cb = rest % ncb;
  const int bh = rest / ncb;
  const long long n_lo = static_cast<long long>(split) * chunk;
  const long long n_hi = n_lo + chunk < N ? n_lo + chunk : N;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int l16 = lane & 15, G = lane >> 4;
  f32x4 acc[NACC][2][RW];
#pragma unroll
  for (int dp = 0; dp < NACC; ++dp)
#pragma unroll
    for (int rt = 0; rt < RW; ++rt) acc[dp][0][rt] = acc[dp][1][rt] = f32x4{0, 0, 0, 0};
  if (n_lo < n_hi) {
    const T* qh = q + (static_cast<long long>(bh) * N) * D;
    const T* lh = dl + (static_cast<long long>(bh) * N) * ldl + cb * CB;
    const int nst = static_cast<int>((n_hi - n_lo + kGemmStep - 1) / kGemmStep);
    auto fetch = [&](int st, T* tQ, T* tL) {
      const long long n0 = n_lo + static_cast<long long>(st) * kGemmStep;
      const int nvalid = static_cast<int>(n_hi - n0);
      DmaQ::issue(tQ, qh + n0 * D, D, nvalid);
      DmaL::issue(tL, lh + n0 * ldl, ldl, nvalid);
    };
    fetch(0, sQ0, sL0);
    __syncthreads();
    auto stage = [&](int st, const T* cQ, const T* cL, T* nQ, T* nL) {
      if (st + 1 < nst) fetch(st + 1, nQ, nL);
      const int nvalid = static_cast<int>(n_hi - (n_lo + static_cast<long long>(st) * kGemmStep));
      typename E::frag vv[NACC][2];
      load_cols<T, D, DK, NACC>(vv, cQ, 0);
      typename E::frag pf[RW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        pf[rt] = Tile<T, CB>::load_tr(cL, 0, (wave * RW + rt) * 16, 4);
        if (nvalid < kGemmStep) {
          // rows past the chunk repeat its last row: zero their slots
          float w[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = 8 * G + j < nvalid ? E::slot(pf[rt], j) : 0.0f;
          pf[rt] = E::pack(w);
        }
      }
      weighted_sum<T, D, NACC, RW>(acc, vv, pf);
      __syncthreads();
    };
    for (int st = 0; st < nst; st += 2) {
      stage(st, sQ0, sL0, sQ1, sL1);
      if (st + 1 < nst) stage(st + 1, sQ1, sL1, sQ0, sL0);
    }
  }
#pragma unroll
  for (int rt = 0; rt < RW; ++rt) {
    const int c1 = cb * CB + (wave * RW + rt) * 16 + l16;
    if (c1 >= b1) continue;
    store_rows<float, D, NACC, RW>(part + ((static_cast<long long>(bh) * nsplit + split) * b1 + c1) * D, acc, rt,
                                   1.0f, G);
  }
}

// -------------------------------------------------------- kb_dkbar_reduce --
// dkbar[bh][c1][:] = (sum over token chunks of the partial sums) / b2: the
// block-mean key gradient spread evenly over the b2 keys of block c1.
template <int D>
__global__ __launch_bounds__(256) void kb_dkbar_reduce(const float* __restrict__ part, float* __restrict__ dkbar,
                                                       int BH, int b1, int b2, int np) {
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long long n = static_cast<long long>(BH) * b1 * (D / 4);
  if (idx >= n) return;
  const int ch = static_cast<int>(idx % (D / 4));
  const long long bc = idx / (D / 4);  // bh*b1 + c1
  const long long bh = bc / b1, c1 = bc % b1;
  f32x4 m = f32x4{0, 0, 0, 0};
  for (int i = 0; i < np; ++i) m += *reinterpret_cast<const f32x4*>(part + ((bh * np + i) * b1 + c1) * D + 4 * ch);
  *reinterpret_cast<f32x4*>(dkbar + bc * D + 4 * ch) = m * (1.0f / static_cast<float>(b2));
}

}  // namespace monarch
