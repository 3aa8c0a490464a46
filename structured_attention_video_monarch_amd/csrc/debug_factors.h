// Test-only kernels: the factors L and R of the last iteration, written out
// from a training forward's stored intermediates (fp32) so that tests can
// compare them with the oracle's element by element.  The layout is the
// oracle's: L[a2][a1][c1] (rows a1 sum to 1 over c1) and R[g][c1][a2][c2]
// (rows sum to 1 over c2); see the MonarchRT article, "Monarch matrices", for
// the factorisation M = P^T L P R.  Plain per-thread dot products: these run
// on small shapes only and are not part of the timed path.
#pragma once

#include "device_common.h"

namespace monarch {

struct FGeom {
  int BH, N, b1, b2, t;
  float c;  // log2(e) / sqrt(d)
};

// tile g of query block a1: tile_lo(g) <= a1 < tile_lo(g + 1)
__device__ inline int tile_of_block(int a1, int b1, int t) {
  int g = 0;
  while (g + 1 < t && tile_lo(g + 1, b1, t) <= a1) ++g;
  return g;
}

// L[bh][a2][a1][c1] = 2^(x - lse_n), x = c <q_n, K[g(a1), c1, a2]> + H (bits),
// n = a1*b2 + a2; K are the block means (first iteration: kt [BH][b1][D],
// h2 NULL) or the keys and entropies of the R-step before ([BH][t][b1][b2]).
template <int D>
__global__ __launch_bounds__(256) void k_factor_L(const float* __restrict__ q, const float* __restrict__ kt,
                                                  const float* __restrict__ h2, const float* __restrict__ lse,
                                                  float* __restrict__ L, FGeom p) {
  const long long per = static_cast<long long>(p.b2) * p.b1 * p.b1;
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= p.BH * per) return;
  const int bh = static_cast<int>(i / per);
  long long r = i % per;
  const int a2 = static_cast<int>(r / (static_cast<long long>(p.b1) * p.b1));
  r %= static_cast<long long>(p.b1) * p.b1;
  const int a1 = static_cast<int>(r / p.b1), c1 = static_cast<int>(r % p.b1);
  const int g = tile_of_block(a1, p.b1, p.t);
  const long long n = static_cast<long long>(bh) * p.N + static_cast<long long>(a1) * p.b2 + a2;
  const long long krow = h2 == nullptr ? static_cast<long long>(bh) * p.b1 + c1
                                       : ((static_cast<long long>(bh) * p.t + g) * p.b1 + c1) * p.b2 + a2;
  const float* qn = q + n * D;
  const float* kr = kt + krow * D;
  float dot = 0.0f;
  for (int j = 0; j < D; ++j) dot = fmaf(qn[j], kr[j], dot);
  const float x = dot * p.c + (h2 == nullptr ? 0.0f : h2[krow]);
  L[i] = exp2f(x - lse[n]);
}

// R[bh][g][c1][a2][c2] = softmax over c2 of c <Qh[g,c1,a2], k_(c1,c2)> (log2
// units), one thread per row (bh, g, c1, a2); the row is written to R first
// as logits, then normalised in place.
template <int D>
__global__ __launch_bounds__(256) void k_factor_R(const float* __restrict__ qhat, const float* __restrict__ k,
                                                  float* __restrict__ R, FGeom p) {
  const long long rows = static_cast<long long>(p.BH) * p.t * p.b1 * p.b2;
  const long long row = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  long long r = row / p.b2;
  const int c1 = static_cast<int>(r % p.b1);
  r /= p.b1;
  const int bh = static_cast<int>(r / p.t);
  const float* qh = qhat + row * D;
  const float* kb = k + (static_cast<long long>(bh) * p.b1 + c1) * p.b2 * D;
  float* out = R + row * p.b2;
  float m = -INFINITY;
  for (int c2 = 0; c2 < p.b2; ++c2) {
    float dot = 0.0f;
    for (int j = 0; j < D; ++j) dot = fmaf(qh[j], kb[static_cast<long long>(c2) * D + j], dot);
    const float x = dot * p.c;
    out[c2] = x;
    m = fmaxf(m, x);
  }
  float sum = 0.0f;
  for (int c2 = 0; c2 < p.b2; ++c2) sum += exp2f(out[c2] - m);
  const float lse = m + log2f(sum);
  for (int c2 = 0; c2 < p.b2; ++c2) out[c2] = exp2f(out[c2] - lse);
}

}  // namespace monarch
