// The backward launch schedule: reverse through the iterations, last to
// first.  Instantiated per I/O type in bwd_bf16.hip / bwd_f32.hip.
#pragma once

#include "backward.h"
#include "backward_cols.h"
#include "backward_long.h"
#include "host.h"

namespace monarch_host {

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
  // the first L-step's keys: block means, stored pre-scaled by c when the
  // forward ran on them so (their logits are then in log2 units already)
  const bool pre = prescaled_keys(s, bf);
  LGeom col_geom1 = col_geom;
  if (pre) col_geom1.c = 1.0f;
  const unsigned col_grid = static_cast<unsigned>(s.BH * s.t * s.b2 * col_geom.nrb);
  // short tile columns (few key blocks, few rows per tile): one column per
  // wave in kb_du and kb_dq
  constexpr int cols_nw = 4;
  const bool cols = s.b1 <= kColsRows && ngmax <= kColsRows;
  const unsigned cols_grid = static_cast<unsigned>(s.BH * s.t * ((s.b2 + cols_nw - 1) / cols_nw));
  // dU = L^T dy per tile column (L of the last L-step); bf16 tiles of at
  // most kColRows rows: the whole column resident in LDS, one workgroup each
  const bool du_col = MONARCH_BDU_COL && sizeof(T) == 2 && !cols && ngmax <= kColRows;
  const unsigned du_col_grid = static_cast<unsigned>(s.BH * s.t * s.b2);
  ok(timed(5, st, [&] {
    if constexpr (sizeof(T) == 2) {
      if (du_col) {
        if (T_ == 1)
          kb_du_col<T, D, MONARCH_BDUC_RW, MONARCH_BDUC_NW, true><<<du_col_grid, MONARCH_BDUC_NW * kWave, 0, st>>>(
              q, dout, bf.kbar, nullptr, bf.lse_of(1), du, col_geom1);
        else
          kb_du_col<T, D, MONARCH_BDUC_RW, MONARCH_BDUC_NW, false><<<du_col_grid, MONARCH_BDUC_NW * kWave, 0, st>>>(
              q, dout, keys_of(T_), ent_of(T_), bf.lse_of(T_), du, col_geom);
        return;
      }
    }
    if (cols && T_ == 1)
      kb_du_cols<T, D, cols_nw, true><<<cols_grid, cols_nw * kWave, 0, st>>>(q, dout, bf.kbar, nullptr, bf.lse_of(1),
                                                                             du, col_geom);
    else if (cols)
      kb_du_cols<T, D, cols_nw, false><<<cols_grid, cols_nw * kWave, 0, st>>>(q, dout, keys_of(T_), ent_of(T_),
                                                                              bf.lse_of(T_), du, col_geom);
    else if (T_ == 1)
      kb_du<T, D, C::kDuRW, C::kDuNW, true><<<col_grid, C::kDuNW * kWave, 0, st>>>(q, dout, bf.kbar, nullptr,
                                                                                  bf.lse_of(1), du, col_geom1);
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
  // kb_rside_a: four waves when each has at least two (tile, row tile) tasks
  // (bf16: three workgroups per CU), else one wave per row tile
  const int ra_ntr = (s.b2 + 15) / 16;
  const int ra_nw = sizeof(T) == 2 && s.t * ra_ntr >= 2 * MONARCH_BRA_NW ? MONARCH_BRA_NW : ra_ntr;
  const unsigned r_threads = static_cast<unsigned>(kWave * ra_nw);
  const unsigned rb_threads =
      static_cast<unsigned>(kWave * (long_blocks ? 8 : (s.b2 + rb_keys - 1) / rb_keys));
  const unsigned rb_grid = static_cast<unsigned>(s.BH * s.b1 * nks);
  const size_t ra_lds = long_blocks ? 0 : rside_bwd_lds_bytes<T, D>(bg.b2p);
  constexpr int ral_nw = 4;
  const RBLGeom ral{BH, s.b1, s.b2, s.t, (s.b2 + 32 * ral_nw - 1) / (32 * ral_nw), c, sc};
  const unsigned ral_grid = static_cast<unsigned>(s.BH * s.b1 * s.t * ral.nrb);
  constexpr int dq_rows = C::kDqRW * C::kDqNW * 16;
  const LGeom row_geom{BH, Nq, s.b1, s.b1q, s.b2, s.t, (ngmax + dq_rows - 1) / dq_rows, c};
  LGeom row_geom1 = row_geom;
  if (pre) row_geom1.c = 1.0f;
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
                                                        ev, dq, dqacc, dl, w.ldl, first ? row_geom1 : row_geom, sc,
                                                        pre && first ? c : 1.0f);
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


}  // namespace monarch_host

#define MONARCH_INSTANTIATE_RUN_BWD(T, D)                                                                   \
  template hipError_t monarch_host::run_bwd<T, D>(const T*, const T*, const T*, const T*, const T*, T*, T*, \
                                                  T*, const Shape&, const Bufs<T>&, unsigned char*,         \
                                                  const BwdWorkspace&, hipStream_t);
