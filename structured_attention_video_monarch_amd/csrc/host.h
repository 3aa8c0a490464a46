// Host-side pieces shared by the library's translation units: the shape of
// a call and its checks, the workspace and training-state layouts, per-launch
// timing, and the tuning knobs of the launch configurations.  The launch
// schedules themselves (run_pass: the forward, run_bwd: the backward) are
// defined in run_fwd.h / run_bwd.h and instantiated once per I/O type in
// their own translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "lside.h"
#include "lside_cols.h"
#include "rside.h"
#include "rside_long.h"
#include "../../include/monarch_attn.h"

namespace monarch_host {
using namespace monarch;


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
// the first L-step's aggregation with the whole tile column in LDS (bf16,
// at most kColRows rows per tile)
#ifndef MONARCH_AGG_COL
#define MONARCH_AGG_COL 1
#endif
#ifndef MONARCH_AGG_SCHED_BARRIER
#define MONARCH_AGG_SCHED_BARRIER 1
#endif
#ifndef MONARCH_APP_SCHED_BARRIER
#define MONARCH_APP_SCHED_BARRIER 1
#endif
#ifndef MONARCH_LSE_SCHED_BARRIER
#define MONARCH_LSE_SCHED_BARRIER 1
#endif


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

inline int check_args(const void* q, const void* k, const void* v, const void* out, const Shape& s,
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

inline Shape make_shape_kv(int B, int H, int fq, int f, int h, int w, int d, int b1, int b2, int t, int T) {
  Shape s{B, H, f, h, w, d, b1, b2, t, T, 0, 0, fq, 0, 0};
  s.N = static_cast<long long>(f) * h * w;
  s.BH = static_cast<long long>(B) * H;
  s.Nq = static_cast<long long>(fq) * h * w;
  s.b1q = b2 > 0 && s.Nq % b2 == 0 ? static_cast<int>(s.Nq / b2) : 0;
  return s;
}

inline Shape make_shape(int B, int H, int f, int h, int w, int d, int b1, int b2, int t, int T) {
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
inline long long heads_per_pass(const Shape& s, size_t elem) {
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

inline Workspace layout(const Shape& s, size_t elem, bool all_heads = false) {
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
extern Profiler g_prof;  // defined with the entry points



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
  // the block means may be stored pre-scaled to log2 units (c Kbar); the
  // backward reads them in the same form (prescaled_keys)
  bool prescale;
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
  b.prescale = true;
  return b;
}

// Whether the first L-step runs on block means pre-scaled by c = log2(e)/sqrt(d)
// (stored so by k_kbar; one multiply-add less per logit): bf16, when the
// buffers allow it and the first L-step's aggregation holds whole tile
// columns (k_aggregate_col); the forward and the backward take the same
// decision from the shape.
template <typename T>
inline bool prescaled_keys(const Shape& s, const Bufs<T>& bf) {
  const long long ngmax0 = (s.b1q + s.t - 1) / s.t;
  return sizeof(T) == 2 && bf.prescale && !(s.b1 <= kColsRows && ngmax0 <= kColsRows) &&
         ngmax0 <= kColRows && MONARCH_AGG_COL;
}

// Early stopping (iterations until the objective stops improving): per-head
// stop iterations (zeroed before the call) and the previous objectives.
struct Adaptive {
  int* stop_at;
  int* nstop_upto;  // [max_iters + 1]: heads stopped after iteration <= i (zeroed before the call)
  double* fprev;
  float tol;
};
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

inline TrainState train_layout(const Shape& s, size_t elem) {
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
  b.prescale = true;
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
// kb_du with the whole tile column in LDS (bf16, at most kColRows rows per
// tile): rows per wave / 16 and waves per workgroup
#ifndef MONARCH_BDU_COL
#define MONARCH_BDU_COL 1
#endif
#ifndef MONARCH_BDUC_RW
#define MONARCH_BDUC_RW 2
#endif
#ifndef MONARCH_BDUC_NW
#define MONARCH_BDUC_NW 8
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

inline BwdWorkspace bwd_layout(const Shape& s, size_t elem) {
  return elem == 2 ? bwd_layout_t<bf16_t>(s) : bwd_layout_t<float>(s);
}

constexpr size_t kLdsBytes = 160 * 1024;

// Workgroups of a launch that loops over `items` work items: a few times as
// many as the chip holds at once (the kernel's occupancy per CU times the
// CUs, times kPersistOver, a multiple of 8 so that every item keeps its XCD),
// and never more than the items.  Each workgroup then takes several items,
// so a launch whose items are all skipped dispatches few workgroups, while
// workgroups still come and go as in a full grid (a CU refills as soon as
// one of its workgroups ends, and the occupancy estimate need not be exact).
constexpr int kPersistOver = 8;
inline unsigned persistent_grid(const void* kernel, int threads, size_t lds, long long items) {
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess || per_cu < 1) {
    (void)hipGetLastError();
    ncu = 256;
    per_cu = 1;
  }
  long long g = static_cast<long long>(ncu) * per_cu * kPersistOver / 8 * 8;
  if (g < 8) g = 8;
  return static_cast<unsigned>(g < items ? g : items);
}

// Launch schedules (forward: run_fwd.h; backward: run_bwd.h).
template <typename T, int D>
hipError_t run_pass(const T* q, const T* k, const T* v, T* out, const Shape& s, const Bufs<T>& bf,
                    hipStream_t st, const Adaptive* ad = nullptr);

template <typename T, int D>
hipError_t run_bwd(const T* q, const T* k, const T* v, const T* out, const T* dout, T* dq, T* dk,
                   T* dv, const Shape& s, const Bufs<T>& bf, unsigned char* ws, const BwdWorkspace& w,
                   hipStream_t st);

}  // namespace monarch_host
