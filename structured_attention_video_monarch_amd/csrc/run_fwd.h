// The forward launch schedule of one pass over a group of heads (block means,
// iters x (L-step, R-step), apply), shared by the plain, early-stopping and
// training forwards.  Instantiated per I/O type in fwd_bf16.hip / fwd_f32.hip.
#pragma once

#include "host.h"

namespace monarch_host {

template <typename T, int D>
hipError_t run_pass(const T* q, const T* k, const T* v, T* out, const Shape& s, const Bufs<T>& bf,
                    hipStream_t st, const Adaptive* ad) {
  const float c = kLog2e / std::sqrt(static_cast<float>(D));
  T* kbar = bf.kbar;
  T* uout = bf.u == bf.qhat ? nullptr : bf.u;
  const int BH = static_cast<int>(s.BH), Nq = static_cast<int>(s.Nq);
  const int ngmax = (s.b1q + s.t - 1) / s.t;  // rows of the largest tile
  hipError_t err = hipSuccess;
  auto ok = [&](hipError_t e) {
    if (e != hipSuccess && err == hipSuccess) err = e;
  };

  // The first L-step's kernels take the block means pre-scaled by c (one
  // multiply-add less per logit) where k_lse, k_aggregate_col and k_apply
  // run them; the training state keeps them in that form for the backward.
  const bool pre = prescaled_keys(s, bf);
  const float cscale = pre ? c : 1.0f;

  // block means of K
  {
    const long long items = s.BH * s.b1;
    const unsigned grid = static_cast<unsigned>((items + 3) / 4);
    if (s.b2 > kShortB2)
      ok(timed(0, st, [&] {
        k_kbar_long<T, D><<<static_cast<unsigned>(items), 256, 0, st>>>(k, kbar, bf.knorm, s.b2, cscale);
      }));
    else
      ok(timed(0, st, [&] { k_kbar<T, D><<<grid, 256, 0, st>>>(k, kbar, bf.knorm, BH, s.b1, s.b2, cscale); }));
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
  // k_aggregate_col: a whole tile column per work item (every key tile)
  LGeom aggc = agg;
  if (MONARCH_AGG_ALLK) aggc.nrb = 1;
  const unsigned aggc_grid = static_cast<unsigned>(s.BH * s.t * s.b2 * aggc.nrb);
  // whole tile column resident in LDS when it is short enough (bf16 only:
  // the f32 column would not fit)
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
    ok(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rstep_adaptive<T, D, true>),
                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(r_lds_last)));
  if (ad && r_lds_mid > 65536)
    ok(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rstep_adaptive<T, D, false>),
                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(r_lds_mid)));
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
    // early stopping, iterations after the first: the iteration's kernels
    // loop over their work items with as many workgroups as the chip holds,
    // skip the heads that stopped before, and return at once when every head
    // has (ns: heads stopped after iteration <= it - 1)
    const bool persist = ad && !first;
    const int* ns = ad ? ad->nstop_upto + (it - 1) : nullptr;
    if (first) {
      ok(timed(1, st, [&] {
        if constexpr (sizeof(T) == 2) {
          if (pre) {
            k_lse<T, D, kLseRW, kLseNW, true, true, true><<<lse_contig_grid, kLseNW * kWave, 0, st>>>(
                q, kbar, nullptr, lse, lse_contig, nullptr, 0, bf.knorm);
            return;
          }
        }
        k_lse<T, D, kLseRW, kLseNW, true, true><<<lse_contig_grid, kLseNW * kWave, 0, st>>>(q, kbar, nullptr, lse, lse_contig,
                                                                                          nullptr, 0, bf.knorm);
      }));
    } else if (persist) {
      auto kern = &k_lse<T, D, kLseRW, kLseNW, false, false>;
      const unsigned grid = persistent_grid(reinterpret_cast<const void*>(kern), kLseNW * kWave, 0, lse_col_grid);
      ok(timed(1, st, [&] {
        kern<<<grid, kLseNW * kWave, 0, st>>>(q, ktil, hent, lse, lse_col, sa, it, nullptr, ns,
                                              static_cast<int>(lse_col_grid));
      }));
    } else {
      ok(timed(1, st, [&] {
        k_lse<T, D, kLseRW, kLseNW, false, false><<<lse_col_grid, kLseNW * kWave, 0, st>>>(q, ktil, hent, lse, lse_col,
                                                                                            sa, it);
      }));
    }
    if (ad) {
      ok(timed(11, st, [&] {
        k_objective<><<<static_cast<unsigned>(s.BH), kObjThreads, 0, st>>>(lse, Nq, s.b2, ad->fprev, ad->stop_at, it,
                                                                          s.T, ad->tol, ad->nstop_upto);
      }));
    }
    if (cols) {
      ok(timed(2, st, [&] {
        if (first)
          k_aggregate_cols<T, D, cols_nw, true><<<cols_grid, cols_nw * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat,
                                                                                     beta, base);
        else if (persist) {
          auto kern = &k_aggregate_cols<T, D, cols_nw, false>;
          const unsigned grid = persistent_grid(reinterpret_cast<const void*>(kern), cols_nw * kWave, 0, cols_grid);
          kern<<<grid, cols_nw * kWave, 0, st>>>(q, ktil, hent, lse, qhat, beta, base, sa, it, ns,
                                                 static_cast<int>(cols_grid));
        } else
          k_aggregate_cols<T, D, cols_nw, false><<<cols_grid, cols_nw * kWave, 0, st>>>(q, ktil, hent, lse, qhat,
                                                                                      beta, base, sa, it);
      }));
    } else if (first) {
      ok(timed(2, st, [&] {
        if constexpr (sizeof(T) == 2) {
          if (pre) {
            k_aggregate_col<T, D, kAggRW, kAggNW, true, true><<<aggc_grid, kAggNW * kWave, 0, st>>>(q, kbar, nullptr, lse,
                                                                                                 qhat, beta, aggc);
            return;
          }
        }
        if (col_fits)
          k_aggregate_col<T, D, kAggRW, kAggNW, true><<<aggc_grid, kAggNW * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat, beta, aggc);
        else
          k_aggregate<T, D, kAggRW, kAggNW, true><<<agg_grid, kAggNW * kWave, 0, st>>>(q, kbar, nullptr, lse, qhat, beta, agg);
      }));
    } else if (persist) {
      ok(timed(2, st, [&] {
        if (col_fits) {
          auto kern = &k_aggregate_col<T, D, kAggRW, kAggNW, false>;
          const unsigned grid = persistent_grid(reinterpret_cast<const void*>(kern), kAggNW * kWave, 0, aggc_grid);
          kern<<<grid, kAggNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, beta, aggc, sa, it, ns,
                                                static_cast<int>(aggc_grid));
        } else {
          auto kern = &k_aggregate<T, D, kAggRW, kAggNW, false>;
          const unsigned grid = persistent_grid(reinterpret_cast<const void*>(kern), kAggNW * kWave, 0, agg_grid);
          kern<<<grid, kAggNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, beta, agg, sa, it, ns,
                                                static_cast<int>(agg_grid));
        }
      }));
    } else {
      ok(timed(2, st, [&] {
        if (col_fits)
          k_aggregate_col<T, D, kAggRW, kAggNW, false><<<aggc_grid, kAggNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, beta,
                                                                                           aggc, sa, it);
        else
          k_aggregate<T, D, kAggRW, kAggNW, false><<<agg_grid, kAggNW * kWave, 0, st>>>(q, ktil, hent, lse, qhat, beta, agg,
                                                                                      sa, it);
      }));
    }
    if (long_blocks) {
      ok(timed(3, st, [&] {
        if (ad) {
          auto kern = &k_rstep_long_adaptive<T, D, kRlRW, kRlNW>;
          const unsigned grid =
              persist ? persistent_grid(reinterpret_cast<const void*>(kern), kRlNW * kWave, 0, rl_grid) : rl_grid;
          kern<<<grid, kRlNW * kWave, 0, st>>>(k, v, qhat, bf.ktil, bf.hent, ad->stop_at, it, rl,
                                               ad->nstop_upto + (it - 1), static_cast<int>(rl_grid));
        }
        else if (bf.rlse) {  // the training forward: fp32 row sums, log-sum-exps kept
          if (last)
            k_rstep_long<T, D, kRlRW, kRlNW, true, true><<<rl_grid, kRlNW * kWave, 0, st>>>(
                k, v, qhat, nullptr, nullptr, uout, bf.rlse_of(it), rl);
          else
            k_rstep_long<T, D, kRlRW, kRlNW, false, true><<<rl_grid, kRlNW * kWave, 0, st>>>(
                k, v, qhat, ktil_out, hent_out, nullptr, bf.rlse_of(it), rl);
        } else if (last)
          k_rstep_long<T, D, kRlRW, kRlNW, true><<<rl_grid, kRlNW * kWave, 0, st>>>(k, v, qhat, nullptr, nullptr,
                                                                                   uout, nullptr, rl);
        else
          k_rstep_long<T, D, kRlRW, kRlNW, false><<<rl_grid, kRlNW * kWave, 0, st>>>(k, v, qhat, ktil_out, hent_out,
                                                                                    nullptr, nullptr, rl);
      }));
    } else if (ad) {
      ok(timed(3, st, [&] {
        // the heads that go on (next keys and entropies), then those that stop now (R V)
        k_rstep_adaptive<T, D, false><<<r_grid, r_threads, r_lds_mid, st>>>(k, v, qhat, bf.ktil, bf.hent, ad->stop_at,
                                                                            it, rg, ad->nstop_upto);
        k_rstep_adaptive<T, D, true><<<r_grid, r_threads, r_lds_last, st>>>(k, v, qhat, bf.ktil, bf.hent, ad->stop_at,
                                                                           it, rg, ad->nstop_upto);
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
      if constexpr (sizeof(T) == 2) {
        if (pre) {
          k_apply<T, D, kAppRW, kAppNW, true, true><<<app_grid, kAppNW * kWave, 0, st>>>(q, kbar, nullptr, lse_last, bf.u,
                                                                                      out, app);
          return;
        }
      }
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


}  // namespace monarch_host

#define MONARCH_INSTANTIATE_RUN_PASS(T, D)                                                              \
  template hipError_t monarch_host::run_pass<T, D>(const T*, const T*, const T*, T*, const Shape&,      \
                                                   const Bufs<T>&, hipStream_t, const Adaptive*);
