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

#include "lside.h"
#include "rside.h"
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

// ------------------------------------------------------------------ checks --
struct Shape {
  int B, H, f, h, w, d, b1, b2, t, T;
  long long N, BH;
};

int check_args(const void* q, const void* k, const void* v, const void* out, const Shape& s,
               size_t elem) {
  if (!q || !k || !v || !out) return MONARCH_EINVAL;
  if (s.B <= 0 || s.H <= 0 || s.f <= 0 || s.h <= 0 || s.w <= 0 || s.d <= 0 || s.b1 <= 0 ||
      s.b2 <= 0)
    return MONARCH_EINVAL;
  const long long N = static_cast<long long>(s.f) * s.h * s.w;
  if (static_cast<long long>(s.b1) * s.b2 != N) return MONARCH_EINVAL;
  if (s.t < 1 || s.t > s.b1) return MONARCH_EINVAL;
  if (s.T < 1) return MONARCH_EINVAL;
  if (s.d != 16 && s.d != 32 && s.d != 64 && s.d != 128) return MONARCH_EUNSUPPORTED;
  if (s.b2 > 128) return MONARCH_EUNSUPPORTED;
  if (static_cast<long long>(s.t) * N * s.d >= (1LL << 31)) return MONARCH_EUNSUPPORTED;
  const long long BH = static_cast<long long>(s.B) * s.H;
  if (BH * s.b1 >= (1LL << 31)) return MONARCH_EUNSUPPORTED;
  // out must not overlap any input
  const uintptr_t bytes = static_cast<uintptr_t>(BH * N * s.d) * elem;
  const uintptr_t o = reinterpret_cast<uintptr_t>(out);
  for (const void* in : {q, k, v}) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(in);
    if (o < a + bytes && a < o + bytes) return MONARCH_EINVAL;
  }
  return MONARCH_OK;
}

Shape make_shape(int B, int H, int f, int h, int w, int d, int b1, int b2, int t, int T) {
  Shape s{B, H, f, h, w, d, b1, b2, t, T, 0, 0};
  s.N = static_cast<long long>(f) * h * w;
  s.BH = static_cast<long long>(B) * H;
  return s;
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
  size_t kbar, lse, qhat, ktil, hent, total;
};

Workspace layout(const Shape& s, size_t elem) {
  Workspace w{};
  w.hc = heads_per_pass(s, elem);
  const size_t hc = static_cast<size_t>(w.hc);
  size_t off = 0;
  w.kbar = off;
  off += align_up(hc * s.b1 * s.d * elem);
  w.lse = off;
  off += align_up(hc * s.N * sizeof(float));
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
    "k_rstep (R block softmax + R V / next keys)", "k_apply (L-apply on the permuted index)"};

// Launch wrapper: records events around the launch when profiling is on.
template <typename F>
hipError_t timed(int id, hipStream_t st, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (g_prof.on) {
    a = g_prof.get();
    b = g_prof.get();
    if (a && b) (void)hipEventRecord(a, st);
  }
  launch();
  hipError_t err = hipGetLastError();
  if (g_prof.on && a && b) {
    (void)hipEventRecord(b, st);
    g_prof.pending.push_back({id, a, b});
  }
  return err;
}

// ------------------------------------------------------------------ launch --
// All kernels of one pass over `s.BH` heads starting at the given pointers.
template <typename T, int D>
hipError_t run_pass(const T* q, const T* k, const T* v, T* out, const Shape& s, unsigned char* ws,
                    const Workspace& w, hipStream_t st) {
  const float c = kLog2e / std::sqrt(static_cast<float>(D));
  T* kbar = reinterpret_cast<T*>(ws + w.kbar);
  float* lse = reinterpret_cast<float*>(ws + w.lse);
  T* qhat = reinterpret_cast<T*>(ws + w.qhat);
  T* ktil = s.T > 1 ? reinterpret_cast<T*>(ws + w.ktil) : nullptr;
  float* hent = s.T > 1 ? reinterpret_cast<float*>(ws + w.hent) : nullptr;
  const int BH = static_cast<int>(s.BH), N = static_cast<int>(s.N);
  const int ngmax = (s.b1 + s.t - 1) / s.t;
  hipError_t err = hipSuccess;
  auto ok = [&](hipError_t e) {
    if (e != hipSuccess && err == hipSuccess) err = e;
  };

  // block means of K
  {
    const long long items = s.BH * s.b1;
    const unsigned grid = static_cast<unsigned>((items + 3) / 4);
    ok(timed(0, st, [&] { k_kbar<T, D><<<grid, 256, 0, st>>>(k, kbar, BH, s.b1, s.b2); }));
  }

  constexpr int lse_rows = kLseRW * kLseNW * 16, agg_rows = kAggRW * kAggNW * 16,
                app_rows = kAppRW * kAppNW * 16;
  const LGeom base{BH, N, s.b1, s.b2, s.t, 0, c};
  LGeom lse_col = base, lse_contig = base, agg = base, app = base;
  lse_col.nrb = (ngmax + lse_rows - 1) / lse_rows;
  lse_contig.nrb = (N + lse_rows - 1) / lse_rows;
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

  RGeom rg{BH, s.b1, s.b2, s.t, (s.b2 + 31) / 32 * 32, c};
  const unsigned r_grid = static_cast<unsigned>(s.BH * s.b1);
  const unsigned r_threads = static_cast<unsigned>(kWave * ((s.b2 + 15) / 16));
  const size_t r_lds_last = rside_lds_bytes<T>(D, rg.b2p, true);
  const size_t r_lds_mid = rside_lds_bytes<T>(D, rg.b2p, false);
  if (r_lds_last > 65536)
    ok(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rstep<T, D, true>),
                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(r_lds_last)));
  if (r_lds_mid > 65536)
    ok(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rstep<T, D, false>),
                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(r_lds_mid)));

  for (int it = 1; it <= s.T; ++it) {
    const bool first = it == 1, last = it == s.T;
    if (first) {
      ok(timed(1, st, [&] {
        k_lse<T, D, kLseRW, kLseNW, true, true><<<lse_contig_grid, kLseNW * kWave, 0, st>>>(q, kbar, nullptr, lse, lse_contig);
      }));
      ok(timed(2, st, [&] {
        if (col_fits)
          k_aggregate_col<T, D, kAggRW, kAggNW, true><<<agg_grid, kAggNW * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat, agg);
        else
          k_aggregate<T, D, kAggRW, kAggNW, true><<<agg_grid, kAggNW * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat, agg);
      }));
    } else {
      ok(timed(1, st, [&] {
        k_lse<T, D, kLseRW, kLseNW, false, false><<<lse_col_grid, kLseNW * kWave, 0, st>>>(q, ktil, hent, lse, lse_col);
      }));
      ok(timed(2, st, [&] {
        if (col_fits)
          k_aggregate_col<T, D, kAggRW, kAggNW, false><<<agg_grid, kAggNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, agg);
        else
          k_aggregate<T, D, kAggRW, kAggNW, false><<<agg_grid, kAggNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, agg);
      }));
    }
    if (last) {
      ok(timed(3, st, [&] {
        k_rstep<T, D, true><<<r_grid, r_threads, r_lds_last, st>>>(k, v, qhat, nullptr, nullptr, rg);
      }));
    } else {
      ok(timed(3, st, [&] {
        k_rstep<T, D, false><<<r_grid, r_threads, r_lds_mid, st>>>(k, v, qhat, ktil, hent, rg);
      }));
    }
  }
  if (s.T == 1) {
    ok(timed(4, st, [&] {
      k_apply<T, D, kAppRW, kAppNW, true><<<app_grid, kAppNW * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat, out, app);
    }));
  } else {
    ok(timed(4, st, [&] {
      k_apply<T, D, kAppRW, kAppNW, false><<<app_grid, kAppNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, out, app);
    }));
  }
  return err;
}

template <typename T, int D>
int run(const T* q, const T* k, const T* v, T* out, const Shape& s, unsigned char* ws,
        const Workspace& w, hipStream_t st) {
  const long long per = s.N * D;
  for (long long h0 = 0; h0 < s.BH; h0 += w.hc) {
    Shape ps = s;
    ps.BH = s.BH - h0 < w.hc ? s.BH - h0 : w.hc;
    const long long o = h0 * per;
    const hipError_t err = run_pass<T, D>(q + o, k + o, v + o, out + o, ps, ws, w, st);
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

}  // namespace

// ------------------------------------------------------------------- C ABI --
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
