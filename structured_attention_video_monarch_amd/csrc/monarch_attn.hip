// Host side of libmonarch_attn.so: the C entry points, argument checks and
// workspaces (the launch schedules are in run_fwd.h and run_bwd.h).
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

#include "debug_factors.h"
#include "host.h"
#include "../../include/monarch_attn.h"

using namespace monarch;
using namespace monarch_host;

namespace monarch_host {
Profiler g_prof;
}  // namespace monarch_host

namespace {

thread_local int g_last_hip_error = 0;

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

// ------------------------------------------------- no-allocation forward --
// The intermediates of monarch_attn_fwd_scratch live in this array, one copy
// per GPU the library's code is loaded on.  In host code its name is only a
// stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress on that GPU (scratch_ptr) and is what the kernels get.
static __device__ __align__(256) unsigned char scratch[MONARCH_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This GPU's copy of the scratch array (looked up once per device, with the
// device current), or nullptr with *err set.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

int fwd_scratch(const void* q, const void* k, const void* v, void* out, const Shape& s, int dtype,
                hipStream_t st) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return MONARCH_EINVAL;
  const int rc = check_args(q, k, v, out, s, elem);
  if (rc != MONARCH_OK) return rc;
  if (layout(s, elem).total > MONARCH_SCRATCH_BYTES) return MONARCH_ENOMEM;
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(&e);
  if (!ws) {
    g_last_hip_error = static_cast<int>(e);
    (void)hipGetLastError();
    return MONARCH_EHIP;
  }
  return fwd_ws(q, k, v, out, s, dtype, ws, MONARCH_SCRATCH_BYTES, st);
}

// --------------------------------------------------- iterate to converge --
// Workspace of the early-stopping call: the forward's for max_iters
// iterations over all heads at once, then the previous objective per head,
// then the counts of heads stopped after each iteration (max_iters + 1 ints).
size_t adaptive_bytes(const Shape& s, size_t elem, size_t* fprev_off, size_t* nstop_off = nullptr) {
  const Workspace w = layout(s, elem, true);
  const size_t f = align_up(static_cast<size_t>(s.BH) * sizeof(double));
  if (fprev_off) *fprev_off = w.total;
  if (nstop_off) *nstop_off = w.total + f;
  return w.total + f + align_up(static_cast<size_t>(s.T + 1) * sizeof(int));
}

int fwd_adaptive(const void* q, const void* k, const void* v, void* out, const Shape& s, int dtype,
                 float tol, int* iters_used, void* workspace, size_t workspace_bytes, hipStream_t st) {
  const size_t elem = elem_size(dtype);
  if (elem == 0) return MONARCH_EINVAL;
  int rc = check_args(q, k, v, out, s, elem);
  if (rc != MONARCH_OK) return rc;
  if (!iters_used || std::isnan(tol)) return MONARCH_EINVAL;
  size_t fprev_off = 0, nstop_off = 0;
  const size_t need = adaptive_bytes(s, elem, &fprev_off, &nstop_off);
  if (!workspace || workspace_bytes < need) return MONARCH_ENOMEM;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return MONARCH_EINVAL;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const Workspace w = layout(s, elem, true);
  int* nstop_upto = reinterpret_cast<int*>(ws + nstop_off);
  Adaptive ad{iters_used, nstop_upto, reinterpret_cast<double*>(ws + fprev_off), tol};
  hipError_t e = hipSuccess;
  clear_stale_error();
  // fill kernels, not memsets: the call can be captured in a HIP graph
  k_fill_int<><<<static_cast<unsigned>((s.BH + 255) / 256), 256, 0, st>>>(iters_used, static_cast<int>(s.BH), 0);
  k_fill_int<><<<static_cast<unsigned>((s.T + 1 + 255) / 256), 256, 0, st>>>(nstop_upto, s.T + 1, 0);
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

int monarch_attn_fwd_scratch(const void* q, const void* k, const void* v, void* out, int B, int H, int f, int h,
                             int w, int d, int b1, int b2, int tiles, int iters, int dtype, void* stream) {
  const Shape s = make_shape(B, H, f, h, w, d, b1, b2, tiles, iters);
  return fwd_scratch(q, k, v, out, s, dtype, static_cast<hipStream_t>(stream));
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
