// Host side of libmonarch_attn.so: argument checks, workspace layout, the
// launch schedule of the kernels, and per-kernel timing.
//
// Schedule for one call (iters = T):
//   k_kbar                          block means of K (R starts uniform)
//   for it = 1..T:
//     k_lse       (L-step)          log2-sum-exp of every L row
//     k_aggregate (R-step, part 1)  Qh = L-weighted mean of each tile's queries
//     k_rstep     (R-step, part 2)  R block softmax, then R V (it = T) or the
//                                   next L-step's keys and entropies (it < T)
//   k_apply                         y = L U on the permuted index
// Kernels of one call run back to back on the caller's stream; nothing
// synchronises with the host.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "backward.h"
#include "backward_long.h"
#include "backward_cols.h"
#include "debug_factors.h"
#include "lside.h"
#include "lside_cols.h"
#include "rside.h"
#include "rside_long.h"
#include "../../include/monarch_attn.h"

using namespace monarch;

namespace {

thread_local int g_last_hip_error = 0;

// ----------------------------------------------------------- tuning knobs --
// Rows per wave (in 16-row MFMA tiles) and waves per workgroup of each
// L-side kernel (overridable at build time for tuning sweeps).
#ifndef MONARCH_LSE_RW
#define MONARCH_LSE_RW 2
#endif
#ifndef MONARCH_LSE_NW
#define MONARCH_LSE_NW 4
#endif
#ifndef MONARCH_AGG_RW
#define MONARCH_AGG_RW 2
#endif
#ifndef MONARCH_AGG_NW
#define MONARCH_AGG_NW 4
#endif
#ifndef MONARCH_APP_RW
#define MONARCH_APP_RW 2
#endif
#ifndef MONARCH_APP_NW
#define MONARCH_APP_NW 4
#endif
constexpr int kLseRW = MONARCH_LSE_RW, kLseNW = MONARCH_LSE_NW;
constexpr int kAggRW = MONARCH_AGG_RW, kAggNW = MONARCH_AGG_NW;
constexpr int kAppRW = MONARCH_APP_RW, kAppNW = MONARCH_APP_NW;
// the R-step of long key blocks (b2 > kShortB2): rows a2 per workgroup
#ifndef MONARCH_RL_RW
#define MONARCH_RL_RW 2
#endif
#ifndef MONARCH_RL_NW
#define MONARCH_RL_NW 4
#endif
constexpr int kRlRW = MONARCH_RL_RW, kRlNW = MONARCH_RL_NW;
// longest key block the forward takes (the long R-step has no limit of its
// own; this bounds the grid and index arithmetic)
constexpr int kMaxB2 = 16384;

// ------------------------------------------------------------------ checks --
// Shapes of one call.  Keys and values: f frames, N = f*h*w tokens in b1
// blocks of b2.  Queries: fq frames, Nq = fq*h*w tokens in b1q blocks of b2
// (fq == f for the square layer; a chunk of frames against cached keys has
// fewer).  Tiles split the query blocks.
struct Shape {
  int B, H, f, h, w, d, b1, b2, t, T;
  long long N, BH;
  int fq, b1q;
  long long Nq;
};

int check_args(const void* q, const void* k, const void* v, const void* out, const Shape& s,
               size_t elem) {
  if (!q || !k || !v || !out) return MONARCH_EINVAL;
  if (s.B <= 0 || s.H <= 0 || s.f <= 0 || s.fq <= 0 || s.h <= 0 || s.w <= 0 || s.d <= 0 ||
      s.b1 <= 0 || s.b2 <= 0)
    return MONARCH_EINVAL;
  const long long N = static_cast<long long>(s.f) * s.h * s.w;
  const long long Nq = static_cast<long long>(s.fq) * s.h * s.w;
  if (static_cast<long long>(s.b1) * s.b2 != N) return MONARCH_EINVAL;
  if (Nq % s.b2 != 0) return MONARCH_EINVAL;
  const long long b1q = Nq / s.b2;
  if (s.t < 1 || s.t > b1q) return MONARCH_EINVAL;
  if (s.T < 1) return MONARCH_EINVAL;
  if (s.d != 16 && s.d != 32 && s.d != 64 && s.d != 128) return MONARCH_EUNSUPPORTED;
  if (s.b2 > kMaxB2) return MONARCH_EUNSUPPORTED;
  if (static_cast<long long>(s.t) * N * s.d >= (1LL << 31)) return MONARCH_EUNSUPPORTED;
  if (Nq * s.d >= (1LL << 31)) return MONARCH_EUNSUPPORTED;
  const long long BH = static_cast<long long>(s.B) * s.H;
  if (BH * s.b1 >= (1LL << 31)) return MONARCH_EUNSUPPORTED;
  // out must not overlap any input
  const uintptr_t qbytes = static_cast<uintptr_t>(BH * Nq * s.d) * elem;
  const uintptr_t kbytes = static_cast<uintptr_t>(BH * N * s.d) * elem;
  const uintptr_t o = reinterpret_cast<uintptr_t>(out);
  const void* ins[3] = {q, k, v};
  const uintptr_t sizes[3] = {qbytes, kbytes, kbytes};
  for (int i = 0; i < 3; ++i) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(ins[i]);
    if (o < a + sizes[i] && a < o + qbytes) return MONARCH_EINVAL;
  }
  return MONARCH_OK;
}

Shape make_shape_kv(int B, int H, int fq, int f, int h, int w, int d, int b1, int b2, int t, int T) {
  Shape s{B, H, f, h, w, d, b1, b2, t, T, 0, 0, fq, 0, 0};
  s.N = static_cast<long long>(f) * h * w;
  s.BH = static_cast<long long>(B) * H;
  s.Nq = static_cast<long long>(fq) * h * w;
  s.b1q = b2 > 0 && s.Nq % b2 == 0 ? static_cast<int>(s.Nq / b2) : 0;
  return s;
}

Shape make_shape(int B, int H, int f, int h, int w, int d, int b1, int b2, int t, int T) {
  return make_shape_kv(B, H, f, f, h, w, d, b1, b2, t, T);
}

// --------------------------------------------------------------- workspace --
constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Heads are processed in passes of `heads_per_pass` (b, h) pairs, all kernels
// of a pass back to back, so that one pass's intermediates (the aggregated
// queries, written over by R V) and its inputs stay in the 256 MB Infinity
// Cache between the kernels that produce and consume them.
// Measured on MI355X at the 720p latent shape: one pass over all heads is
// faster than per-head passes (launch tails outweigh cache residency), so the
// default budget is unlimited (0); a budget bounds the workspace instead.
#ifndef MONARCH_PASS_BUDGET_MB
#define MONARCH_PASS_BUDGET_MB 0
#endif
long long heads_per_pass(const Shape& s, size_t elem) {
  if (MONARCH_PASS_BUDGET_MB <= 0) return s.BH;
  const long long nd = s.N * s.d * static_cast<long long>(elem);
  long long per_head = s.t * nd + 4 * nd + s.N * 4;
  if (s.T > 1) per_head += s.t * nd + s.t * s.N * 4;
  const long long budget = static_cast<long long>(MONARCH_PASS_BUDGET_MB) << 20;
  long long hc = budget / per_head;
  if (hc < 1) hc = 1;
  if (hc > s.BH) hc = s.BH;
  return hc;
}

struct Workspace {
  long long hc;  // heads per pass
  size_t kbar, knorm, lse, qhat, ktil, hent, total;
};

Workspace layout(const Shape& s, size_t elem, bool all_heads = false) {
  Workspace w{};
  w.hc = all_heads ? s.BH : heads_per_pass(s, elem);
  const size_t hc = static_cast<size_t>(w.hc);
  size_t off = 0;
  w.kbar = off;
  off += align_up(hc * s.b1 * s.d * elem);
  w.knorm = off;
  off += align_up(hc * s.b1 * sizeof(float));
  w.lse = off;
  off += align_up(hc * s.Nq * sizeof(float));
  w.qhat = off;
  off += align_up(hc * s.t * s.N * s.d * elem);
  if (s.T > 1) {
    w.ktil = off;
    off += align_up(hc * s.t * s.N * s.d * elem);
    w.hent = off;
    off += align_up(hc * s.t * s.N * sizeof(float));
  } else {
    w.ktil = w.hent = 0;
  }
  w.total = off;
  return w;
}

// ---------------------------------------------------------------- profiling --
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  struct Rec { int id; hipEvent_t a, b; };
  std::vector<Rec> pending;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler g_prof;

const char* const kKernelNames[MONARCH_NUM_KERNELS] = {
    "k_kbar (block-mean keys)", "k_lse (L-row log-sum-exp)", "k_aggregate (R-side aggregation through L)",
    "k_rstep (R block softmax + R V / next keys)", "k_apply (L-apply on the permuted index)",
    "kb_du (backward: dU = L^T dy per tile column)",
    "kb_rside_a (backward: R-step per key block, G and row statistics)",
    "kb_dq (backward: row pass, dq)", "kb_dkbar (backward: block-mean key gradient over tokens)",
    "kb_dkbar_reduce (backward: sum of the token-chunk partials)",
    "kb_rside_b (backward: dv and dk per key block)",
    "k_objective (objective per head and the early-stop decision)",
    "kb_dktil (backward: gradient of the aggregated keys and entropies per tile column)"};

// The HIP runtime's last-error slot is per thread and shared with every other
// user of the runtime in the process (a framework that loaded the same
// runtime may leave an error there); clear it before a launch so that the
// check after the launch sees only that launch's error.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Launch wrapper: records events around the launch when profiling is on.
// The profiler's state (switch, event pool, pending records) is shared by
// every thread that launches through the library, so it is only touched with
// its lock held; the launch itself runs outside the lock.
template <typename F>
hipError_t timed(int id, hipStream_t st, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.on) {
      a = g_prof.get();
      b = g_prof.get();
      if (!a || !b) {  // no event pair: this launch goes untimed
        if (a) g_prof.pool.push_back(a);
        if (b) g_prof.pool.push_back(b);
        a = b = nullptr;
      }
    }
  }
  if (a) (void)hipEventRecord(a, st);
  clear_stale_error();
  launch();
  hipError_t err = hipGetLastError();
  if (a) {
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.pending.push_back({id, a, b});
  }
  return err;
}

// ------------------------------------------------------------------ launch --
// All kernels of one pass over `s.BH` heads starting at the given pointers.
// Intermediates of one pass.  `u` receives R V (== qhat: written over the
// aggregated queries); `beta` receives the column masses when not NULL (both
// kept for the backward pass by the training forward).  The *_it strides
// (elements) place each iteration's log-sum-exps, masses, aggregated queries
// and next keys/entropies in a copy of its own, as the backward pass through
// several iterations needs; 0 writes every iteration over the same buffer.
template <typename T>
struct Bufs {
  T* kbar;
  float* knorm;  // |Kbar| per key block (offsets of the first L-step's log-sum-exp)
  float* lse;
  T* qhat;
  T* ktil;
  float* hent;
  T* u;
  float* beta;
  float* rlse;  // training with key blocks over 128: the R rows' log-sum-exps
  long long lse_it, qhat_it, beta_it, ktil_it, hent_it;
  // views of iteration it (1-based); keys/entropies: those the R-step of
  // iteration it writes (it < T), read by the L-step of it + 1
  float* lse_of(int it) const { return lse + (it - 1) * lse_it; }
  T* qhat_of(int it) const { return qhat + (it - 1) * qhat_it; }
  float* beta_of(int it) const { return beta ? beta + (it - 1) * beta_it : nullptr; }
  T* ktil_of(int it) const { return ktil ? ktil + (it - 1) * ktil_it : nullptr; }
  float* hent_of(int it) const { return hent ? hent + (it - 1) * hent_it : nullptr; }
  float* rlse_of(int it) const { return rlse ? rlse + (it - 1) * beta_it : nullptr; }
};

template <typename T>
Bufs<T> bufs_of(const Shape& s, unsigned char* ws, const Workspace& w) {
  Bufs<T> b{};
  b.kbar = reinterpret_cast<T*>(ws + w.kbar);
  b.knorm = reinterpret_cast<float*>(ws + w.knorm);
  b.lse = reinterpret_cast<float*>(ws + w.lse);
  b.qhat = reinterpret_cast<T*>(ws + w.qhat);
  b.ktil = s.T > 1 ? reinterpret_cast<T*>(ws + w.ktil) : nullptr;
  b.hent = s.T > 1 ? reinterpret_cast<float*>(ws + w.hent) : nullptr;
  b.u = b.qhat;
  b.beta = nullptr;
  b.rlse = nullptr;
  return b;
}

// Early stopping (iterations until the objective stops improving): per-head
// stop iterations (zeroed before the call) and the previous objectives.
struct Adaptive {
  int* stop_at;
  double* fprev;
  float tol;
};

template <typename T, int D>
hipError_t run_pass(const T* q, const T* k, const T* v, T* out, const Shape& s, const Bufs<T>& bf,
                    hipStream_t st, const Adaptive* ad = nullptr) {
  const float c = kLog2e / std::sqrt(static_cast<float>(D));
  T* kbar = bf.kbar;
  T* uout = bf.u == bf.qhat ? nullptr : bf.u;
  const int BH = static_cast<int>(s.BH), Nq = static_cast<int>(s.Nq);
  const int ngmax = (s.b1q + s.t - 1) / s.t;  // rows of the largest tile
  hipError_t err = hipSuccess;
  auto ok = [&](hipError_t e) {
    if (e != hipSuccess && err == hipSuccess) err = e;
  };

  // block means of K
  {
    const long long items = s.BH * s.b1;
    const unsigned grid = static_cast<unsigned>((items + 3) / 4);
    if (s.b2 > kShortB2)
      ok(timed(0, st, [&] {
        k_kbar_long<T, D><<<static_cast<unsigned>(items), 256, 0, st>>>(k, kbar, bf.knorm, s.b2);
      }));
    else
      ok(timed(0, st, [&] { k_kbar<T, D><<<grid, 256, 0, st>>>(k, kbar, bf.knorm, BH, s.b1, s.b2); }));
  }

  constexpr int lse_rows = kLseRW * kLseNW * 16, agg_rows = kAggRW * kAggNW * 16,
                app_rows = kAppRW * kAppNW * 16;
  const LGeom base{BH, Nq, s.b1, s.b1q, s.b2, s.t, 0, c};
  LGeom lse_col = base, lse_contig = base, agg = base, app = base;
  lse_col.nrb = (ngmax + lse_rows - 1) / lse_rows;
  lse_contig.nrb = (Nq + lse_rows - 1) / lse_rows;
  agg.nrb = (s.b1 + agg_rows - 1) / agg_rows;
  app.nrb = (ngmax + app_rows - 1) / app_rows;
  const unsigned lse_col_grid = static_cast<unsigned>(s.BH * s.t * s.b2 * lse_col.nrb);
  const unsigned lse_contig_grid = static_cast<unsigned>(s.BH * lse_contig.nrb);
  const unsigned app_grid = static_cast<unsigned>(s.BH * s.t * s.b2 * app.nrb);
  const unsigned agg_grid = static_cast<unsigned>(s.BH * s.t * s.b2 * agg.nrb);
  // whole tile column resident in LDS when it is short enough (bf16 only:
  // the f32 column would not fit)
#ifndef MONARCH_AGG_COL
#define MONARCH_AGG_COL 1
#endif
  const bool col_fits = MONARCH_AGG_COL && sizeof(T) == 2 && ngmax <= kColRows;
  // short tile columns (few key blocks, few rows per tile, e.g. blocks of
  // whole frames): one column per wave
  constexpr int cols_nw = 4;
  const bool cols = s.b1 <= kColsRows && ngmax <= kColsRows;
  const unsigned cols_grid = static_cast<unsigned>(s.BH * s.t * ((s.b2 + cols_nw - 1) / cols_nw));

  // R-step: a whole block row per wave (b2 <= kShortB2), else the online
  // softmax over blocks of 64 keys with RB rows a2 per workgroup
  const bool long_blocks = s.b2 > kShortB2;
  RGeom rg{BH, s.b1, s.b2, s.t, (s.b2 + 31) / 32 * 32, c};
  const unsigned r_grid = static_cast<unsigned>(s.BH * s.b1);
  const unsigned r_threads = static_cast<unsigned>(kWave * ((s.b2 + 15) / 16));
  const size_t r_lds_last = long_blocks ? 0 : rside_lds_bytes<T>(D, rg.b2p, true);
  const size_t r_lds_mid = long_blocks ? 0 : rside_lds_bytes<T>(D, rg.b2p, false);
  constexpr int rl_rows = kRlRW * kRlNW * 16;
  RLGeom rl{BH, s.b1, s.b2, s.t, (s.b2 + rl_rows - 1) / rl_rows, c};
  const unsigned rl_grid = static_cast<unsigned>(s.BH * s.b1 * s.t * rl.nrb);
  if (r_lds_last > 65536)
    ok(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rstep<T, D, true>),
                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(r_lds_last)));
  if (r_lds_mid > 65536)
    ok(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rstep<T, D, false>),
                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(r_lds_mid)));

  const int* sa = ad ? ad->stop_at : nullptr;
  if (ad && r_lds_last > 65536)
    ok(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rstep_adaptive<T, D>),
                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(r_lds_last)));
  for (int it = 1; it <= s.T; ++it) {
    const bool first = it == 1, last = it == s.T;
    float* lse = bf.lse_of(it);
    T* qhat = bf.qhat_of(it);
    float* beta = bf.beta_of(it);
    // keys and entropies this L-step reads, and those this R-step writes
    const T* ktil = first ? nullptr : bf.ktil_of(it - 1);
    const float* hent = first ? nullptr : bf.hent_of(it - 1);
    T* ktil_out = last ? nullptr : bf.ktil_of(it);
    float* hent_out = last ? nullptr : bf.hent_of(it);
    if (first) {
      ok(timed(1, st, [&] {
        k_lse<T, D, kLseRW, kLseNW, true, true><<<lse_contig_grid, kLseNW * kWave, 0, st>>>(q, kbar, nullptr, lse, lse_contig,
                                                                                          nullptr, 0, bf.knorm);
      }));
    } else {
      ok(timed(1, st, [&] {
        k_lse<T, D, kLseRW, kLseNW, false, false><<<lse_col_grid, kLseNW * kWave, 0, st>>>(q, ktil, hent, lse, lse_col,
                                                                                            sa, it);
      }));
    }
    if (ad) {
      ok(timed(11, st, [&] {
        k_objective<<<static_cast<unsigned>(s.BH), 256, 0, st>>>(lse, Nq, s.b2, ad->fprev, ad->stop_at, it, s.T,
                                                                  ad->tol);
      }));
    }
    if (cols) {
      ok(timed(2, st, [&] {
        if (first)
          k_aggregate_cols<T, D, cols_nw, true><<<cols_grid, cols_nw * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat,
                                                                                     beta, base);
        else
          k_aggregate_cols<T, D, cols_nw, false><<<cols_grid, cols_nw * kWave, 0, st>>>(q, ktil, hent, lse, qhat,
                                                                                      beta, base, sa, it);
      }));
    } else if (first) {
      ok(timed(2, st, [&] {
        if (col_fits)
          k_aggregate_col<T, D, kAggRW, kAggNW, true><<<agg_grid, kAggNW * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat, beta, agg);
        else
          k_aggregate<T, D, kAggRW, kAggNW, true><<<agg_grid, kAggNW * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat, beta, agg);
      }));
    } else {
      ok(timed(2, st, [&] {
        if (col_fits)
          k_aggregate_col<T, D, kAggRW, kAggNW, false><<<agg_grid, kAggNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, beta, agg,
                                                                                          sa, it);
        else
          k_aggregate<T, D, kAggRW, kAggNW, false><<<agg_grid, kAggNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, beta, agg,
                                                                                      sa, it);
      }));
    }
    if (long_blocks) {
      ok(timed(3, st, [&] {
        if (ad)
          k_rstep_long_adaptive<T, D, kRlRW, kRlNW><<<rl_grid, kRlNW * kWave, 0, st>>>(k, v, qhat, bf.ktil, bf.hent,
                                                                                      ad->stop_at, it, rl);
        else if (last)
          k_rstep_long<T, D, kRlRW, kRlNW, true><<<rl_grid, kRlNW * kWave, 0, st>>>(k, v, qhat, nullptr, nullptr,
                                                                                   uout, bf.rlse_of(it), rl);
        else
          k_rstep_long<T, D, kRlRW, kRlNW, false><<<rl_grid, kRlNW * kWave, 0, st>>>(k, v, qhat, ktil_out, hent_out,
                                                                                    nullptr, bf.rlse_of(it), rl);
      }));
    } else if (ad) {
      ok(timed(3, st, [&] {
        k_rstep_adaptive<T, D><<<r_grid, r_threads, r_lds_last, st>>>(k, v, qhat, bf.ktil, bf.hent, ad->stop_at, it,
                                                                       rg);
      }));
    } else if (last) {
      ok(timed(3, st, [&] {
        k_rstep<T, D, true><<<r_grid, r_threads, r_lds_last, st>>>(k, v, qhat, nullptr, nullptr, uout, rg);
      }));
    } else {
      ok(timed(3, st, [&] {
        k_rstep<T, D, false><<<r_grid, r_threads, r_lds_mid, st>>>(k, v, qhat, ktil_out, hent_out, nullptr, rg);
      }));
    }
  }
  const float* lse_last = bf.lse_of(s.T);
  if (cols) {
    ok(timed(4, st, [&] {
      if (s.T == 1)
        k_apply_cols<T, D, cols_nw, true><<<cols_grid, cols_nw * kWave, 0, st>>>(q, kbar, nullptr, lse_last, bf.u,
                                                                               out, base);
      else
        k_apply_cols<T, D, cols_nw, false><<<cols_grid, cols_nw * kWave, 0, st>>>(
            q, bf.ktil_of(s.T - 1), bf.hent_of(s.T - 1), lse_last, bf.u, out, base);
    }));
  } else if (s.T == 1) {
    ok(timed(4, st, [&] {
      k_apply<T, D, kAppRW, kAppNW, true><<<app_grid, kAppNW * kWave, 0, st>>>(q, kbar, nullptr, lse_last, bf.u, out,
                                                                              app);
    }));
  } else {
    const T* kt = bf.ktil_of(s.T - 1);
    const float* ht = bf.hent_of(s.T - 1);
    ok(timed(4, st, [&] {
      k_apply<T, D, kAppRW, kAppNW, false><<<app_grid, kAppNW * kWave, 0, st>>>(q, kt, ht, lse_last, bf.u, out, app);
    }));
  }
  return err;
}

template <typename T, int D>
int run(const T* q, const T* k, const T* v, T* out, const Shape& s, unsigned char* ws,
        const Workspace& w, hipStream_t st) {
  for (long long h0 = 0; h0 < s.BH; h0 += w.hc) {
    Shape ps = s;
    ps.BH = s.BH - h0 < w.hc ? s.BH - h0 : w.hc;
    const long long oq = h0 * s.Nq * D, ok = h0 * s.N * D;
    const hipError_t err =
        run_pass<T, D>(q + oq, k + ok, v + ok, out + oq, ps, bufs_of<T>(ps, ws, w), st);
    if (err != hipSuccess) {
      g_last_hip_error = static_cast<int>(err);
      return MONARCH_EHIP;
    }
  }
  return MONARCH_OK;
}

template <typename T>
int dispatch(const void* q, const void* k, const void* v, void* out, const Shape& s,
             unsigned char* ws, const Workspace& w, hipStream_t st) {
  const T* tq = static_cast<const T*>(q);
  const T* tk = static_cast<const T*>(k);
  const T* tv = static_cast<const T*>(v);
  T* to = static_cast<T*>(out);
  switch (s.d) {
    case 16: return run<T, 16>(tq, tk, tv, to, s, ws, w, st);
    case 32: return run<T, 32>(tq, tk, tv, to, s, ws, w, st);
    case 64: return run<T, 64>(tq, tk, tv, to, s, ws, w, st);
    case 128: return run<T, 128>(tq, tk, tv, to, s, ws, w, st);
    default: return MONARCH_EUNSUPPORTED;
  }
}

size_t elem_size(int dtype) {
  return dtype == MONARCH_BF16 ? 2 : dtype == MONARCH_F32 ? 4 : 0;
}

int fwd_ws(const void* q, const void* k, const void* v, void* out, const Shape& s, int dtype,
           void* workspace, size_t workspace_bytes, hipStream_t st) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return MONARCH_EINVAL;
  int rc = check_args(q, k, v, out, s, elem);
  if (rc != MONARCH_OK) return rc;
  const Workspace w = layout(s, elem);
  if (!workspace || workspace_bytes < w.total) return MONARCH_ENOMEM;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return MONARCH_EINVAL;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (dtype == MONARCH_BF16) return dispatch<bf16_t>(q, k, v, out, s, ws, w, st);
  return dispatch<float>(q, k, v, out, s, ws, w, st);
}

int fwd_alloc(const void* q, const void* k, const void* v, void* out, const Shape& s, int dtype,
              hipStream_t st) {
  const size_t elem = elem_size(dtype);
  int rc = check_args(q, k, v, out, s, elem);
  if (rc != MONARCH_OK) return rc;
  const Workspace w = layout(s, elem);
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, w.total, st);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? MONARCH_ENOMEM : MONARCH_EHIP;
  }
  rc = fwd_ws(q, k, v, out, s, dtype, ws, w.total, st);
  e = hipFreeAsync(ws, st);
  if (rc == MONARCH_OK && e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    rc = MONARCH_EHIP;
  }
  return rc;
}

// --------------------------------------------------- iterate to converge --
// Workspace of the early-stopping call: the forward's for max_iters
// iterations over all heads at once, then the previous objective per head.
size_t adaptive_bytes(const Shape& s, size_t elem, size_t* fprev_off) {
  const Workspace w = layout(s, elem, true);
  if (fprev_off) *fprev_off = w.total;
  return w.total + align_up(static_cast<size_t>(s.BH) * sizeof(double));
}

int fwd_adaptive(const void* q, const void* k, const void* v, void* out, const Shape& s, int dtype,
                 float tol, int* iters_used, void* workspace, size_t workspace_bytes, hipStream_t st) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return MONARCH_EINVAL;
  int rc = check_args(q, k, v, out, s, elem);
  if (rc != MONARCH_OK) return rc;
  if (!iters_used || std::isnan(tol)) return MONARCH_EINVAL;
  size_t fprev_off = 0;
  const size_t need = adaptive_bytes(s, elem, &fprev_off);
  if (!workspace || workspace_bytes < need) return MONARCH_ENOMEM;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return MONARCH_EINVAL;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const Workspace w = layout(s, elem, true);
  Adaptive ad{iters_used, reinterpret_cast<double*>(ws + fprev_off), tol};
  hipError_t e = hipSuccess;
  clear_stale_error();
  k_fill_int<<<static_cast<unsigned>((s.BH + 255) / 256), 256, 0, st>>>(iters_used, static_cast<int>(s.BH), 0);
  e = hipGetLastError();
  auto go = [&](auto tag) {
    using T = decltype(tag);
    const Bufs<T> b = bufs_of<T>(s, ws, w);
    const T* tq = static_cast<const T*>(q);
    const T* tk = static_cast<const T*>(k);
    const T* tv = static_cast<const T*>(v);
    T* to = static_cast<T*>(out);
    switch (s.d) {
      case 16: e = run_pass<T, 16>(tq, tk, tv, to, s, b, st, &ad); break;
      case 32: e = run_pass<T, 32>(tq, tk, tv, to, s, b, st, &ad); break;
      case 64: e = run_pass<T, 64>(tq, tk, tv, to, s, b, st, &ad); break;
      default: e = run_pass<T, 128>(tq, tk, tv, to, s, b, st, &ad); break;
    }
  };
  if (e == hipSuccess) {
    if (dtype == MONARCH_BF16) go(bf16_t{}); else go(float{});
  }
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return MONARCH_EHIP;
  }
  return MONARCH_OK;
}

// ------------------------------------------------------------ training --
// Training state: what the backward pass reads from the forward, for all
// heads of the call: the block means, and per iteration i = 1..T the L-row
// log-sum-exps, the column masses and the aggregated queries; U = R V of the
// last R-step; for i < T the keys and entropies the R-step of i hands to the
// next L-step.  Each per-iteration array holds T (or T - 1) copies, one
// aligned block apart.
struct TrainState {
  size_t kbar, knorm, lse, beta, qhat, u, ktil, hent, rlse, total;
  size_t lse_blk, beta_blk, qhat_blk, hent_blk;  // bytes per iteration copy
};

TrainState train_layout(const Shape& s, size_t elem) {
  TrainState t{};
  const size_t BH = static_cast<size_t>(s.BH), N = static_cast<size_t>(s.N), d = static_cast<size_t>(s.d);
  const size_t Nq = static_cast<size_t>(s.Nq);
  const size_t tN = static_cast<size_t>(s.t) * N;
  const size_t T = static_cast<size_t>(s.T);
  t.lse_blk = align_up(BH * Nq * sizeof(float));
  t.beta_blk = align_up(BH * tN * sizeof(float));
  t.qhat_blk = align_up(BH * tN * d * elem);
  t.hent_blk = t.beta_blk;
  size_t off = 0;
  t.kbar = off;
  off += align_up(BH * s.b1 * d * elem);
  t.knorm = off;
  off += align_up(BH * s.b1 * sizeof(float));
  t.lse = off;
  off += T * t.lse_blk;
  t.beta = off;
  off += T * t.beta_blk;
  t.qhat = off;
  off += T * t.qhat_blk;
  t.u = off;
  off += t.qhat_blk;
  t.ktil = off;
  off += (T - 1) * t.qhat_blk;
  t.hent = off;
  off += (T - 1) * t.hent_blk;
  // key blocks over 128: every R-step's row log-sum-exps (the backward's
  // key-block pass takes them instead of a pass over the block of its own)
  t.rlse = off;
  if (s.b2 > kShortB2) off += T * t.beta_blk;
  t.total = off;
  return t;
}

template <typename T>
Bufs<T> train_bufs(unsigned char* st, const TrainState& t, int iters) {
  Bufs<T> b{};
  b.kbar = reinterpret_cast<T*>(st + t.kbar);
  b.knorm = reinterpret_cast<float*>(st + t.knorm);
  b.lse = reinterpret_cast<float*>(st + t.lse);
  b.qhat = reinterpret_cast<T*>(st + t.qhat);
  b.ktil = iters > 1 ? reinterpret_cast<T*>(st + t.ktil) : nullptr;
  b.hent = iters > 1 ? reinterpret_cast<float*>(st + t.hent) : nullptr;
  b.u = reinterpret_cast<T*>(st + t.u);
  b.beta = reinterpret_cast<float*>(st + t.beta);
  b.rlse = t.rlse < t.total ? reinterpret_cast<float*>(st + t.rlse) : nullptr;
  b.lse_it = static_cast<long long>(t.lse_blk / sizeof(float));
  b.beta_it = static_cast<long long>(t.beta_blk / sizeof(float));
  b.qhat_it = static_cast<long long>(t.qhat_blk / sizeof(T));
  b.ktil_it = b.qhat_it;
  b.hent_it = static_cast<long long>(t.hent_blk / sizeof(float));
  return b;
}

// Backward tuning: rows/keys per wave (16-wide tiles) and waves per
// workgroup of each backward kernel.
template <typename T> struct BwdCfg;
#ifndef MONARCH_BDQ_RW
#define MONARCH_BDQ_RW 2
#endif
#ifndef MONARCH_BDQ_NW
#define MONARCH_BDQ_NW 8
#endif
#ifndef MONARCH_BDQ_STEP
#define MONARCH_BDQ_STEP 64
#endif
#ifndef MONARCH_BRBL_RW
#define MONARCH_BRBL_RW 2  // keys per wave / 16 of kb_rside_b for key blocks over 128
#endif
#ifndef MONARCH_BDU_RW
#define MONARCH_BDU_RW 1
#endif
#ifndef MONARCH_BDU_NW
#define MONARCH_BDU_NW 8
#endif
#ifndef MONARCH_BGM_RW
#define MONARCH_BGM_RW 4
#endif
#ifndef MONARCH_BGM_NW
#define MONARCH_BGM_NW 4
#endif
template <> struct BwdCfg<bf16_t> {
  static constexpr int kDuRW = MONARCH_BDU_RW, kDuNW = MONARCH_BDU_NW;
  static constexpr int kDqRW = MONARCH_BDQ_RW, kDqNW = MONARCH_BDQ_NW, kDqStep = MONARCH_BDQ_STEP;
  static constexpr int kGmRW = MONARCH_BGM_RW, kGmNW = MONARCH_BGM_NW;
};
template <> struct BwdCfg<float> {
  static constexpr int kDuRW = 1, kDuNW = 4, kDqRW = 1, kDqNW = 4, kDqStep = 64, kGmRW = 2, kGmNW = 4;
};

// Backward workspace (allocated per call, stream-ordered).  With several
// iterations `du` also carries dKt of each earlier R-step, `dh` its dH, and
// dq, dk add up in fp32 (dqacc, dkacc).
struct BwdWorkspace {
  int ldl;          // row stride of the stored s*dl (keys padded to the product's key block)
  int nsplit, chunk;  // split of the tokens in the key-mean product
  size_t du, gq, ev, lser, rho, dl, part, dkbar, dh, dqacc, dkacc, total;
};

template <typename T>
BwdWorkspace bwd_layout_t(const Shape& s) {
  using C = BwdCfg<T>;
  constexpr int cb = C::kGmRW * C::kGmNW * 16;
  // kb_dktil reads whole blocks of its own key width from the padded rows
  static_assert(cb % (C::kDuRW * C::kDuNW * 16) == 0, "key blocks of kb_dktil must tile ldl");
  BwdWorkspace w{};
  const size_t elem = sizeof(T);
  const long long ncb = (s.b1 + cb - 1) / cb;
  w.ldl = static_cast<int>(ncb * cb);
  // enough workgroups to fill the chip, chunks of at least 512 query tokens
  long long ns = (2048 + s.BH * ncb - 1) / (s.BH * ncb);
  const long long ns_max = (s.Nq + 511) / 512;
  if (ns > ns_max) ns = ns_max;
  if (ns < 1) ns = 1;
  long long chunk = (s.Nq + ns - 1) / ns;
  chunk = (chunk + 31) / 32 * 32;
  w.nsplit = static_cast<int>((s.Nq + chunk - 1) / chunk);
  w.chunk = static_cast<int>(chunk);
  // query-side buffers have Nq rows, key-side ones t*N (per tile and key block)
  const size_t BH = static_cast<size_t>(s.BH), N = static_cast<size_t>(s.N), d = static_cast<size_t>(s.d);
  const size_t Nq = static_cast<size_t>(s.Nq);
  const size_t tN = static_cast<size_t>(s.t) * N;
  size_t off = 0;
  w.du = off;
  off += align_up(BH * tN * d * elem);
  w.gq = off;
  off += align_up(BH * tN * d * elem);
  w.ev = off;
  off += align_up(BH * tN * sizeof(float));
  w.lser = off;
  off += align_up(BH * tN * sizeof(float));
  w.rho = off;
  off += align_up(BH * tN * sizeof(float));
  w.dl = off;
  off += align_up(BH * Nq * static_cast<size_t>(w.ldl) * elem);
  w.part = off;
  off += align_up(BH * static_cast<size_t>(w.nsplit) * s.b1 * d * sizeof(float));
  w.dkbar = off;
  off += align_up(BH * static_cast<size_t>(s.b1) * d * sizeof(float));
  if (s.T > 1) {
    w.dh = off;
    off += align_up(BH * tN * sizeof(float));
    w.dqacc = off;
    off += align_up(BH * Nq * d * sizeof(float));
    w.dkacc = off;
    off += align_up(BH * N * d * sizeof(float));
  }
  w.total = off;
  return w;
}

BwdWorkspace bwd_layout(const Shape& s, size_t elem) {
  return elem == 2 ? bwd_layout_t<bf16_t>(s) : bwd_layout_t<float>(s);
}

constexpr size_t kLdsBytes = 160 * 1024;

// Reverse through the iterations, last to first.  Per iteration i:
//   R-step part 1 (G, e, row statistics), row pass (dq term, s*dl),
//   R-step part 2 (dv at i = T; the dk terms), then the key side of the
//   L-step: dKt, dH of the R-step before (i > 1) or the block-mean gradient
//   (i = 1).  The last iteration's cotangents come from dy through the apply
//   (dU); an earlier one's from the next L-step (dKt, dH).
template <typename T, int D>
hipError_t run_bwd(const T* q, const T* k, const T* v, const T* out, const T* dout, T* dq, T* dk,
                   T* dv, const Shape& s, const Bufs<T>& bf, unsigned char* ws, const BwdWorkspace& w,
                   hipStream_t st) {
  using C = BwdCfg<T>;
  const float c = kLog2e / std::sqrt(static_cast<float>(D));
  const float sc = 1.0f / std::sqrt(static_cast<float>(D));
  T* du = reinterpret_cast<T*>(ws + w.du);
  T* gq = reinterpret_cast<T*>(ws + w.gq);
  float* ev = reinterpret_cast<float*>(ws + w.ev);
  float* lser = reinterpret_cast<float*>(ws + w.lser);
  float* rho = reinterpret_cast<float*>(ws + w.rho);
  T* dl = reinterpret_cast<T*>(ws + w.dl);
  float* part = reinterpret_cast<float*>(ws + w.part);
  float* dkbar = reinterpret_cast<float*>(ws + w.dkbar);
  float* dh = s.T > 1 ? reinterpret_cast<float*>(ws + w.dh) : nullptr;
  float* dqacc = s.T > 1 ? reinterpret_cast<float*>(ws + w.dqacc) : nullptr;
  float* dkacc = s.T > 1 ? reinterpret_cast<float*>(ws + w.dkacc) : nullptr;
  // the row-side kernels see the Nq query tokens in b1q blocks (tiles split
  // them); key blocks are b1
  const int BH = static_cast<int>(s.BH), N = static_cast<int>(s.N), Nq = static_cast<int>(s.Nq);
  const int ngmax = (s.b1q + s.t - 1) / s.t;
  const int T_ = s.T;
  hipError_t err = hipSuccess;
  auto ok = [&](hipError_t e) {
    if (e != hipSuccess && err == hipSuccess) err = e;
  };
  // keys and entropies of the L-step of iteration i
  auto keys_of = [&](int i) -> const T* { return i == 1 ? bf.kbar : bf.ktil_of(i - 1); };
  auto ent_of = [&](int i) -> const float* { return i == 1 ? nullptr : bf.hent_of(i - 1); };

  constexpr int du_cb = C::kDuRW * C::kDuNW * 16;
  const LGeom col_geom{BH, Nq, s.b1, s.b1q, s.b2, s.t, (s.b1 + du_cb - 1) / du_cb, c};
  const unsigned col_grid = static_cast<unsigned>(s.BH * s.t * s.b2 * col_geom.nrb);
  // short tile columns (few key blocks, few rows per tile): one column per
  // wave in kb_du and kb_dq
  constexpr int cols_nw = 4;
  const bool cols = s.b1 <= kColsRows && ngmax <= kColsRows;
  const unsigned cols_grid = static_cast<unsigned>(s.BH * s.t * ((s.b2 + cols_nw - 1) / cols_nw));
  // dU = L^T dy per tile column (L of the last L-step)
  ok(timed(5, st, [&] {
    if (cols && T_ == 1)
      kb_du_cols<T, D, cols_nw, true><<<cols_grid, cols_nw * kWave, 0, st>>>(q, dout, bf.kbar, nullptr, bf.lse_of(1),
                                                                             du, col_geom);
    else if (cols)
      kb_du_cols<T, D, cols_nw, false><<<cols_grid, cols_nw * kWave, 0, st>>>(q, dout, keys_of(T_), ent_of(T_),
                                                                              bf.lse_of(T_), du, col_geom);
    else if (T_ == 1)
      kb_du<T, D, C::kDuRW, C::kDuNW, true><<<col_grid, C::kDuNW * kWave, 0, st>>>(q, dout, bf.kbar, nullptr,
                                                                                  bf.lse_of(1), du, col_geom);
    else
      kb_du<T, D, C::kDuRW, C::kDuNW, false><<<col_grid, C::kDuNW * kWave, 0, st>>>(
          q, dout, keys_of(T_), ent_of(T_), bf.lse_of(T_), du, col_geom);
  }));

  // key-block kernels: a whole block row per wave (b2 <= kShortB2), else
  // the row statistics taken online over 64-key steps (kb_rside_a_long) and
  // the block's keys in slices of 8 waves (kb_rside_b)
  const bool long_blocks = s.b2 > kShortB2;
  constexpr int rb_keys = 16 * MONARCH_BRB_RW;  // keys c2 per wave of kb_rside_b
  constexpr int rbl_keys = 16 * MONARCH_BRBL_RW;  // keys per wave of kb_rside_b for long blocks
  const int nks = long_blocks ? (s.b2 + 8 * rbl_keys - 1) / (8 * rbl_keys) : 1;
  const BGeom bg{BH, N, s.b1, s.b2, s.t, (s.b2 + 31) / 32 * 32, c, sc, nks, 8 * rbl_keys};
  const unsigned r_grid = static_cast<unsigned>(s.BH * s.b1);
  const unsigned r_threads = static_cast<unsigned>(kWave * ((s.b2 + 15) / 16));
  const unsigned rb_threads =
      static_cast<unsigned>(kWave * (long_blocks ? 8 : (s.b2 + rb_keys - 1) / rb_keys));
  const unsigned rb_grid = static_cast<unsigned>(s.BH * s.b1 * nks);
  const size_t ra_lds = long_blocks ? 0 : rside_bwd_lds_bytes<T, D>(bg.b2p);
  constexpr int ral_nw = 4;
  const RBLGeom ral{BH, s.b1, s.b2, s.t, (s.b2 + 32 * ral_nw - 1) / (32 * ral_nw), c, sc};
  const unsigned ral_grid = static_cast<unsigned>(s.BH * s.b1 * s.t * ral.nrb);
  constexpr int dq_rows = C::kDqRW * C::kDqNW * 16;
  const LGeom row_geom{BH, Nq, s.b1, s.b1q, s.b2, s.t, (ngmax + dq_rows - 1) / dq_rows, c};
  const unsigned row_grid = static_cast<unsigned>(s.BH * s.t * s.b2 * row_geom.nrb);

  for (int i = T_; i >= 1; --i) {
    const bool last = i == T_, first = i == 1;
    const T* qh = bf.qhat_of(i);
    const float* bt = bf.beta_of(i);
    // R-step backward per key block, part 1: G, e and the R row statistics
    if (long_blocks) {
      ok(timed(6, st, [&] {
        // the R rows' lse from the forward; rho from U (last R-step) or from
        // the keys Kt and entropies H this R-step handed to the next L-step
        if (last)
          kb_rside_a_long<T, D, ral_nw, false><<<ral_grid, ral_nw * kWave, 0, st>>>(
              k, v, qh, du, dh, bt, bf.rlse_of(i), bf.u, nullptr, gq, ev, lser, rho, ral);
        else
          kb_rside_a_long<T, D, ral_nw, true><<<ral_grid, ral_nw * kWave, 0, st>>>(
              k, v, qh, du, dh, bt, bf.rlse_of(i), bf.ktil_of(i), bf.hent_of(i), gq, ev, lser, rho, ral);
      }));
    } else {
      auto launch = [&](auto kern) {
        if (ra_lds > 65536)
          ok(hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 static_cast<int>(ra_lds)));
        ok(timed(6, st, [&] {
          kern<<<r_grid, r_threads, ra_lds, st>>>(k, v, qh, du, dh, bt, gq, ev, lser, rho, bg);
        }));
      };
      const int ncp = bg.b2p / 32;
      if (last) {
        switch (ncp) {
          case 1: launch(&kb_rside_a<T, D, 1, false>); break;
          case 2: launch(&kb_rside_a<T, D, 2, false>); break;
          case 3: launch(&kb_rside_a<T, D, 3, false>); break;
          default: launch(&kb_rside_a<T, D, 4, false>); break;
        }
      } else {
        switch (ncp) {
          case 1: launch(&kb_rside_a<T, D, 1, true>); break;
          case 2: launch(&kb_rside_a<T, D, 2, true>); break;
          case 3: launch(&kb_rside_a<T, D, 3, true>); break;
          default: launch(&kb_rside_a<T, D, 4, true>); break;
        }
      }
    }
    // row pass: this L-step's dq term and the stored s*dl
    if (cols) {
      // f32 tiles are twice as large: two columns per workgroup
      constexpr int dq_nw = sizeof(T) == 2 ? cols_nw : 2;
      const unsigned dq_grid = static_cast<unsigned>(s.BH * s.t * ((s.b2 + dq_nw - 1) / dq_nw));
      auto launch = [&](auto kern) {
        ok(timed(7, st, [&] {
          kern<<<dq_grid, dq_nw * kWave, 0, st>>>(q, dout, out, keys_of(i), ent_of(i), bf.lse_of(i), bf.u, gq, ev,
                                                  dq, dqacc, dl, w.ldl, row_geom, sc);
        }));
      };
      if (T_ == 1)
        launch(&kb_dq_cols<T, D, dq_nw, true, true, kDqStore>);
      else if (last)
        launch(&kb_dq_cols<T, D, dq_nw, false, true, kDqInit>);
      else if (first)
        launch(&kb_dq_cols<T, D, dq_nw, true, false, kDqFinish>);
      else
        launch(&kb_dq_cols<T, D, dq_nw, false, false, kDqAdd>);
    } else {
      auto launch = [&](auto kern) {
        ok(timed(7, st, [&] {
          kern<<<row_grid, C::kDqNW * kWave, 0, st>>>(q, dout, out, keys_of(i), ent_of(i), bf.lse_of(i), bf.u, gq,
                                                        ev, dq, dqacc, dl, w.ldl, row_geom, sc);
        }));
      };
      constexpr int RW = C::kDqRW, NW = C::kDqNW, SP = C::kDqStep;
      if (T_ == 1)
        launch(&kb_dq<T, D, RW, NW, true, true, kDqStore, SP>);
      else if (last)
        launch(&kb_dq<T, D, RW, NW, false, true, kDqInit, SP>);
      else if (first)
        launch(&kb_dq<T, D, RW, NW, true, false, kDqFinish, SP>);
      else
        launch(&kb_dq<T, D, RW, NW, false, false, kDqAdd, SP>);
    }
    if (first) {
      // block-mean key gradient: partial sums over chunks of tokens, then
      // their sum spread over the b2 keys of each block
      constexpr int cb = C::kGmRW * C::kGmNW * 16;
      const int ncb = w.ldl / cb;
      const unsigned grid = static_cast<unsigned>(s.BH * ncb * w.nsplit);
      ok(timed(8, st, [&] {
        kb_dkbar<T, D, C::kGmRW, C::kGmNW><<<grid, C::kGmNW * kWave, 0, st>>>(q, dl, w.ldl, part, BH, Nq, s.b1, ncb,
                                                                             w.nsplit, w.chunk);
      }));
      const long long threads = s.BH * s.b1 * (D / 4);
      const unsigned rgrid = static_cast<unsigned>((threads + 255) / 256);
      ok(timed(9, st, [&] { kb_dkbar_reduce<D><<<rgrid, 256, 0, st>>>(part, dkbar, BH, s.b1, s.b2, w.nsplit); }));
    }
    // R-step backward per key block, part 2: dv (last R-step) and the dk terms
    {
      auto launch = [&](auto kern) {
        ok(timed(10, st, [&] {
          kern<<<rb_grid, rb_threads, 0, st>>>(k, v, qh, du, lser, rho, dh, dkbar, dk, dkacc, dv, bg);
        }));
      };
      constexpr int RL = MONARCH_BRBL_RW;
      if (long_blocks) {
        if (T_ == 1)
          launch(&kb_rside_b<T, D, kRbSingle, RL>);
        else if (last)
          launch(&kb_rside_b<T, D, kRbLast, RL>);
        else if (first)
          launch(&kb_rside_b<T, D, kRbFirst, RL>);
        else
          launch(&kb_rside_b<T, D, kRbMid, RL>);
      } else if (T_ == 1) {
        launch(&kb_rside_b<T, D, kRbSingle>);
      } else if (last) {
        launch(&kb_rside_b<T, D, kRbLast>);
      } else if (first) {
        launch(&kb_rside_b<T, D, kRbFirst>);
      } else {
        launch(&kb_rside_b<T, D, kRbMid>);
      }
    }
    // key side of an L-step on aggregated keys: dKt and dH of the R-step
    // before, into du and dh (their last readers, this iteration's R-step
    // kernels, have run)
    if (!first) {
      ok(timed(12, st, [&] {
        kb_dktil<T, D, C::kDuRW, C::kDuNW><<<col_grid, C::kDuNW * kWave, 0, st>>>(q, dl, w.ldl, du, dh, col_geom,
                                                                                 1.0f / sc);
      }));
    }
  }
  return err;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_train(const Shape& s, size_t elem, const void* state, size_t state_bytes) {
  if (elem == 0) return MONARCH_EINVAL;
  const TrainState t = train_layout(s, elem);
  if (!state || state_bytes < t.total) return MONARCH_ENOMEM;
  if (reinterpret_cast<uintptr_t>(state) % kAlign != 0) return MONARCH_EINVAL;
  return MONARCH_OK;
}

int fwd_train(const void* q, const void* k, const void* v, void* out, const Shape& s, int dtype,
              void* state, size_t state_bytes, hipStream_t st) {
  const size_t elem = elem_size(dtype);
  int rc = check_args(q, k, v, out, s, elem);
  if (rc != MONARCH_OK) return rc;
  rc = check_train(s, elem, state, state_bytes);
  if (rc != MONARCH_OK) return rc;
  const size_t qio = static_cast<size_t>(s.BH * s.Nq * s.d) * elem;
  const size_t kio = static_cast<size_t>(s.BH * s.N * s.d) * elem;
  const void* ios[] = {q, k, v, out};
  const size_t iosz[] = {qio, kio, kio, qio};
  for (int i = 0; i < 4; ++i)
    if (overlaps(ios[i], iosz[i], state, state_bytes)) return MONARCH_EINVAL;
  const TrainState t = train_layout(s, elem);
  unsigned char* sp = static_cast<unsigned char*>(state);
  hipError_t e = hipSuccess;
  auto go = [&](auto tag) {
    using T = decltype(tag);
    const Bufs<T> b = train_bufs<T>(sp, t, s.T);
    const T* tq = static_cast<const T*>(q);
    const T* tk = static_cast<const T*>(k);
    const T* tv = static_cast<const T*>(v);
    T* to = static_cast<T*>(out);
    switch (s.d) {
      case 16: e = run_pass<T, 16>(tq, tk, tv, to, s, b, st); break;
      case 32: e = run_pass<T, 32>(tq, tk, tv, to, s, b, st); break;
      case 64: e = run_pass<T, 64>(tq, tk, tv, to, s, b, st); break;
      default: e = run_pass<T, 128>(tq, tk, tv, to, s, b, st); break;
    }
  };
  if (dtype == MONARCH_BF16) go(bf16_t{}); else go(float{});
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return MONARCH_EHIP;
  }
  return MONARCH_OK;
}

int bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, void* dq,
        void* dk, void* dv, const Shape& s, int dtype, void* state, size_t state_bytes, hipStream_t st) {
  const size_t elem = elem_size(dtype);
  int rc = check_args(q, k, v, out, s, elem);
  if (rc != MONARCH_OK) return rc;
  if (!dout || !dq || !dk || !dv) return MONARCH_EINVAL;
  rc = check_train(s, elem, state, state_bytes);
  if (rc != MONARCH_OK) return rc;
  // q, out, dout and dq have Nq rows per head; k, v, dk and dv N
  const size_t qio = static_cast<size_t>(s.BH * s.Nq * s.d) * elem;
  const size_t kio = static_cast<size_t>(s.BH * s.N * s.d) * elem;
  const void* ins[] = {q, k, v, out, dout, state};
  const size_t insz[] = {qio, kio, kio, qio, qio, state_bytes};
  void* outs[] = {dq, dk, dv};
  const size_t outsz[] = {qio, kio, kio};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return MONARCH_EINVAL;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return MONARCH_EINVAL;
  }
  const int b2p = (s.b2 + 31) / 32 * 32;
  const int DK = s.d < 32 ? 32 : s.d;
  if (s.b2 <= kShortB2 && static_cast<size_t>(b2p) * DK * elem * 2 > kLdsBytes) return MONARCH_EUNSUPPORTED;

  const TrainState t = train_layout(s, elem);
  const BwdWorkspace w = bwd_layout(s, elem);
  void* wsp = nullptr;
  hipError_t e = hipMallocAsync(&wsp, w.total, st);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? MONARCH_ENOMEM : MONARCH_EHIP;
  }
  unsigned char* ws = static_cast<unsigned char*>(wsp);
  unsigned char* sp = static_cast<unsigned char*>(state);
  auto go = [&](auto tag) {
    using T = decltype(tag);
    const Bufs<T> b = train_bufs<T>(sp, t, s.T);
    const T* a[5] = {static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<const T*>(out), static_cast<const T*>(dout)};
    T* g3[3] = {static_cast<T*>(dq), static_cast<T*>(dk), static_cast<T*>(dv)};
    switch (s.d) {
      case 16: e = run_bwd<T, 16>(a[0], a[1], a[2], a[3], a[4], g3[0], g3[1], g3[2], s, b, ws, w, st); break;
      case 32: e = run_bwd<T, 32>(a[0], a[1], a[2], a[3], a[4], g3[0], g3[1], g3[2], s, b, ws, w, st); break;
      case 64: e = run_bwd<T, 64>(a[0], a[1], a[2], a[3], a[4], g3[0], g3[1], g3[2], s, b, ws, w, st); break;
      default: e = run_bwd<T, 128>(a[0], a[1], a[2], a[3], a[4], g3[0], g3[1], g3[2], s, b, ws, w, st); break;
    }
  };
  if (dtype == MONARCH_BF16) go(bf16_t{}); else go(float{});
  const hipError_t ef = hipFreeAsync(wsp, st);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return MONARCH_EHIP;
  }
  return MONARCH_OK;
}

}  // namespace

// ------------------------------------------------------------------- C ABI --
// The factors of the last iteration (test-only export): a fp32 training
// forward into a stream-ordered temporary state, then L and R written from
// its lse, keys, entropies and aggregated queries.
int debug_factors(const float* q, const float* k, const float* v, float* L_out, float* R_out, const Shape& s,
                  hipStream_t st) {
  if (!q || !k || !v || !L_out || !R_out) return MONARCH_EINVAL;
  static const char dummy[4] = {0};
  int rc = check_args(dummy, dummy + 1, dummy + 2, dummy + 3, s, 0);  // shape checks
  if (rc != MONARCH_OK) return rc;
  const long long lcount = s.BH * s.b2 * static_cast<long long>(s.b1) * s.b1;
  const long long rcount = s.BH * s.t * s.N * static_cast<long long>(s.b2);
  if (lcount > (1LL << 28) || rcount > (1LL << 28)) return MONARCH_EUNSUPPORTED;
  const size_t io = static_cast<size_t>(s.BH * s.N * s.d) * sizeof(float);
  const void* ins[] = {q, k, v};
  void* outs[] = {L_out, R_out};
  const size_t outsz[] = {static_cast<size_t>(lcount) * sizeof(float), static_cast<size_t>(rcount) * sizeof(float)};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], io)) return MONARCH_EINVAL;
  if (overlaps(L_out, outsz[0], R_out, outsz[1])) return MONARCH_EINVAL;

  const TrainState t = train_layout(s, sizeof(float));
  void* tmp = nullptr;
  hipError_t e = hipMallocAsync(&tmp, t.total + io, st);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? MONARCH_ENOMEM : MONARCH_EHIP;
  }
  unsigned char* state = static_cast<unsigned char*>(tmp);
  float* y = reinterpret_cast<float*>(state + t.total);
  rc = fwd_train(q, k, v, y, s, MONARCH_F32, state, t.total, st);
  if (rc == MONARCH_OK) {
    const Bufs<float> b = train_bufs<float>(state, t, s.T);
    const FGeom fg{static_cast<int>(s.BH), static_cast<int>(s.N), s.b1, s.b2, s.t,
                   kLog2e / std::sqrt(static_cast<float>(s.d))};
    const float* kt = s.T == 1 ? b.kbar : b.ktil_of(s.T - 1);
    const float* h2 = s.T == 1 ? nullptr : b.hent_of(s.T - 1);
    const unsigned lgrid = static_cast<unsigned>((lcount + 255) / 256);
    const unsigned rgrid = static_cast<unsigned>((s.BH * s.t * s.N + 255) / 256);
    auto go = [&](auto dtag) {
      constexpr int D = decltype(dtag)::value;
      k_factor_L<D><<<lgrid, 256, 0, st>>>(q, kt, h2, b.lse_of(s.T), L_out, fg);
      k_factor_R<D><<<rgrid, 256, 0, st>>>(b.qhat_of(s.T), k, R_out, fg);
    };
    switch (s.d) {
      case 16: go(std::integral_constant<int, 16>{}); break;
      case 32: go(std::integral_constant<int, 32>{}); break;
      case 64: go(std::integral_constant<int, 64>{}); break;
      default: go(std::integral_constant<int, 128>{}); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) {
      g_last_hip_error = static_cast<int>(e);
      rc = MONARCH_EHIP;
    }
  }
  const hipError_t ef = hipFreeAsync(tmp, st);
  if (rc == MONARCH_OK && ef != hipSuccess) {
    g_last_hip_error = static_cast<int>(ef);
    rc = MONARCH_EHIP;
  }
  return rc;
}

extern "C" {

int monarch_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int f,
                     int h, int w, int d, int b1, int b2, int tiles, int iters, void* stream) {
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  return fwd_alloc(q, k, v, out, s, MONARCH_BF16, static_cast<hipStream_t>(stream));
}

int monarch_attn_fwd_f32(const float* q, const float* k, const float* v, float* out, int B, int H,
                         int f, int h, int w, int d, int b1, int b2, int tiles, int iters,
                         void* stream) {
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  return fwd_alloc(q, k, v, out, s, MONARCH_F32, static_cast<hipStream_t>(stream));
}

size_t monarch_attn_workspace_bytes(int B, int H, int f, int h, int w, int d, int b1, int b2,
                                    int tiles, int iters, int dtype) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return 0;
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  // shape checks only (pointers are not known here)
  static const char dummy[4] = {0};
  const int rc = check_args(dummy, dummy + 1, dummy + 2, dummy + 3, s, 0);
  if (rc != MONARCH_OK) return 0;
  return layout(s, elem).total;
}

int monarch_attn_fwd_ws(const void* q, const void* k, const void* v, void* out, int B, int H,
                        int f, int h, int w, int d, int b1, int b2, int tiles, int iters,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  return fwd_ws(q, k, v, out, s, dtype, workspace, workspace_bytes,
                static_cast<hipStream_t>(stream));
}

size_t monarch_attn_adaptive_workspace_bytes(int B, int H, int f, int h, int w, int d, int b1, int b2,
                                             int tiles, int max_iters, int dtype) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return 0;
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, max_iters);
  static const char dummy[4] = {0};
  if (check_args(dummy, dummy + 1, dummy + 2, dummy + 3, s, 0) != MONARCH_OK) return 0;
  return adaptive_bytes(s, elem, nullptr);
}

int monarch_attn_fwd_adaptive_ws(const void* q, const void* k, const void* v, void* out, int B, int H,
                                 int f, int h, int w, int d, int b1, int b2, int tiles, int max_iters,
                                 float tol, int dtype, int* iters_used, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, max_iters);
  return fwd_adaptive(q, k, v, out, s, dtype, tol, iters_used, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream));
}

size_t monarch_attn_adaptive_kv_workspace_bytes(int B, int H, int fq, int f, int h, int w, int d, int b1, int b2,
                                                int tiles, int max_iters, int dtype) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return 0;
  const Shape s = make_shape_kv(B, H, fq, f, h, w, d, b1, b2, tiles, max_iters);
  static const char dummy[4] = {0};
  if (check_args(dummy, dummy + 1, dummy + 2, dummy + 3, s, 0) != MONARCH_OK) return 0;
  return adaptive_bytes(s, elem, nullptr);
}

int monarch_attn_fwd_adaptive_kv_ws(const void* q, const void* k, const void* v, void* out, int B, int H, int fq,
                                    int f, int h, int w, int d, int b1, int b2, int tiles, int max_iters,
                                    float tol, int dtype, int* iters_used, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const Shape s = make_shape_kv(B, H, fq, f, h, w, d, b1, b2, tiles, max_iters);
  return fwd_adaptive(q, k, v, out, s, dtype, tol, iters_used, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream));
}

size_t monarch_attn_kv_workspace_bytes(int B, int H, int fq, int f, int h, int w, int d, int b1, int b2,
                                       int tiles, int iters, int dtype) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return 0;
  const Shape s = make_shape_kv(B, H, fq, f, h, w, d, b1, b2, tiles, iters);
  static const char dummy[4] = {0};
  if (check_args(dummy, dummy + 1, dummy + 2, dummy + 3, s, 0) != MONARCH_OK) return 0;
  return layout(s, elem).total;
}

int monarch_attn_fwd_kv(const void* q, const void* k, const void* v, void* out, int B, int H, int fq,
                        int f, int h, int w, int d, int b1, int b2, int tiles, int iters, int dtype,
                        void* stream) {
  const Shape s = make_shape_kv(B, H, fq, f, h, w, d, b1, b2, tiles, iters);
  if (elem_size(dtype) == 0) return MONARCH_EINVAL;
  return fwd_alloc(q, k, v, out, s, dtype, static_cast<hipStream_t>(stream));
}

int monarch_attn_fwd_kv_ws(const void* q, const void* k, const void* v, void* out, int B, int H,
                           int fq, int f, int h, int w, int d, int b1, int b2, int tiles, int iters,
                           int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const Shape s = make_shape_kv(B, H, fq, f, h, w, d, b1, b2, tiles, iters);
  return fwd_ws(q, k, v, out, s, dtype, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

size_t monarch_attn_train_state_bytes(int B, int H, int f, int h, int w, int d, int b1, int b2,
                                      int tiles, int iters, int dtype) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return 0;
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  static const char dummy[4] = {0};
  if (check_args(dummy, dummy + 1, dummy + 2, dummy + 3, s, 0) != MONARCH_OK) return 0;
  return train_layout(s, elem).total;
}

int monarch_attn_fwd_train(const void* q, const void* k, const void* v, void* out, int B, int H,
                           int f, int h, int w, int d, int b1, int b2, int tiles, int iters, int dtype,
                           void* state, size_t state_bytes, void* stream) {
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  return fwd_train(q, k, v, out, s, dtype, state, state_bytes, static_cast<hipStream_t>(stream));
}

int monarch_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     void* dq, void* dk, void* dv, int B, int H, int f, int h, int w, int d, int b1,
                     int b2, int tiles, int iters, int dtype, void* state, size_t state_bytes, void* stream) {
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  return bwd(q, k, v, out, dout, dq, dk, dv, s, dtype, state, state_bytes,
             static_cast<hipStream_t>(stream));
}

size_t monarch_attn_train_state_bytes_kv(int B, int H, int fq, int f, int h, int w, int d, int b1, int b2,
                                         int tiles, int iters, int dtype) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return 0;
  const Shape s = make_shape_kv(B, H, fq, f, h, w, d, b1, b2, tiles, iters);
  static const char dummy[4] = {0};
  if (check_args(dummy, dummy + 1, dummy + 2, dummy + 3, s, 0) != MONARCH_OK) return 0;
  return train_layout(s, elem).total;
}

int monarch_attn_fwd_train_kv(const void* q, const void* k, const void* v, void* out, int B, int H, int fq,
                              int f, int h, int w, int d, int b1, int b2, int tiles, int iters, int dtype,
                              void* state, size_t state_bytes, void* stream) {
  const Shape s = make_shape_kv(B, H, fq, f, h, w, d, b1, b2, tiles, iters);
  return fwd_train(q, k, v, out, s, dtype, state, state_bytes, static_cast<hipStream_t>(stream));
}

int monarch_attn_bwd_kv(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        void* dq, void* dk, void* dv, int B, int H, int fq, int f, int h, int w, int d,
                        int b1, int b2, int tiles, int iters, int dtype, void* state, size_t state_bytes,
                        void* stream) {
  const Shape s = make_shape_kv(B, H, fq, f, h, w, d, b1, b2, tiles, iters);
  return bwd(q, k, v, out, dout, dq, dk, dv, s, dtype, state, state_bytes, static_cast<hipStream_t>(stream));
}

int monarch_attn_debug_factors_f32(const float* q, const float* k, const float* v, float* L_out, float* R_out,
                                   int B, int H, int f, int h, int w, int d, int b1, int b2, int tiles, int iters,
                                   void* stream) {
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  return debug_factors(q, k, v, L_out, R_out, s, static_cast<hipStream_t>(stream));
}

const char* monarch_attn_status_string(int status) {
  switch (status) {
    case MONARCH_OK: return "ok";
    case MONARCH_EINVAL: return "invalid argument";
    case MONARCH_EUNSUPPORTED: return "unsupported shape (outside the kernels' envelope)";
    case MONARCH_EHIP: return "HIP runtime error";
    case MONARCH_ENOMEM: return "workspace allocation failed or workspace too small";
    default: return "unknown status";
  }
}

int monarch_attn_last_hip_error(void) { return g_last_hip_error; }

int monarch_attn_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = on != 0;
  return MONARCH_OK;
}

int monarch_attn_profile_collect(double* ms, long* launches, int n) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  int rc = MONARCH_OK;
  for (auto& r : g_prof.pending) {
    float t = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) {
      g_last_hip_error = static_cast<int>(e);
      rc = MONARCH_EHIP;
    } else if (r.id < n) {
      if (ms) ms[r.id] += t;
      if (launches) launches[r.id] += 1;
    }
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.pending.clear();
  return rc;
}

const char* monarch_attn_kernel_name(int id) {
  if (id < 0 || id >= MONARCH_NUM_KERNELS) return "unknown";
  return kKernelNames[id];
}

}  // extern "C"
