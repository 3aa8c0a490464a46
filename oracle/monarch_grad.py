"""CPU oracle for the gradient of the tiled MonarchAttention forward
(float64 numpy), through one or several unrolled iterations.

TEST INFRASTRUCTURE, like monarch_oracle: only the tests, the smoke check and
the benchmark's CPU baseline may import or call it.

Why a gradient: the pages' main regime is one refinement iteration after the
video model has been finetuned with the attention in place (yunpan.plus
MonarchRT article, "Innovation 3: finetuning and efficient kernels",
Fig. 4 right; atlas.scime.ai summary, "Approach").  Finetuning needs
dL/dQ, dL/dK, dL/dV of the layer.  The pages give no formula for it, so it is
the chain rule applied to the forward as monarch_oracle computes it for one
iteration, written out step by step in reverse:

  forward (R starts uniform, so the L-step keys are the block means Kbar and
  the entropy term log(b2) is the same for every block and cancels):
    Kbar[c1]     = mean_c2 k_(c1,c2)
    L[a2][a1,:]  = softmax_c1( s <q_(a1,a2), Kbar[c1]> )
    beta         = sum_(a1 in g) L,   Qhat = sum_(a1 in g) L q / beta
    R[g,c1,a2,:] = softmax_c2( s <Qhat[g,c1,a2], k_(c1,c2)> )
    U[g,c1,a2]   = sum_c2 R v_(c1,c2)
    y_(a1,a2)    = sum_c1 L[a2][a1,c1] U[g(a1),c1,a2]

  reverse, given dy:
    dL  = <dy, U>                     dU = sum_(a1 in g) L dy
    dR  = <dU, v>                     dv += sum_(g,a2) R dU
    dz  = R (dR - sum_c2 R dR)        (softmax backward, z the R logits)
    dQhat = s sum_c2 dz k             dk += s sum_(g,a2) dz Qhat
    G   = dQhat / beta  (0 where beta == 0, matching Qhat := 0 there)
    dL += <G, q - Qhat>               dq += sum_c1 L G
    dl  = L (dL - sum_c1 L dL)        (softmax backward, l the L logits)
    dq += s sum_c1 dl Kbar            dKbar = s sum_n dl q_n
    dk += dKbar / b2                  (the block mean)

With several iterations the reverse also runs back through the earlier
ones (see monarch_head_grad).  A chunk of query frames against cached keys
(fewer query blocks b1q than key blocks b1, as in monarch_oracle) takes the
same steps with a1 over the chunk's blocks and c1 over all key blocks.
Pinned by central finite differences of the forward oracle, by the block
shapes where the method is exact softmax attention, by symmetries of the
forward, and for a chunk by the square layer's gradient (tests).
"""
from __future__ import annotations

import math

import numpy as np

from .monarch_oracle import _blocks, l_step, r_step, tile_bounds, uniform_R

__all__ = ["monarch_head_grad", "monarch_attention_grad"]


def monarch_head_grad(q, k, v, dy, b1: int, b2: int, tiles: int = 1, iters: int = 1):
    """Gradient of sum(dy * y) for one (batch, head) after ``iters`` iterations.

    q, dy: [Nq, d]; k, v: [N, d] with N = b1*b2 and Nq a multiple of b2
    (Nq = N for the square layer, fewer rows for a chunk against cached keys;
    tiles split the b1q = Nq/b2 query blocks).  Returns (dq [Nq, d],
    dk [N, d], dv [N, d]) float64.

    For iters > 1 the reverse also runs through the earlier iterations: the
    L-step of iteration i uses the keys Kt_(i-1) = R_(i-1) k and entropies
    H_(i-1) = H(R_(i-1)) of the R-step before it, so its logit gradient dl_i
    gives dKt_(i-1) = s sum_(a1 in g) dl_i q and dH_(i-1) = sum_(a1 in g) dl_i,
    and from those dR_(i-1) = <dKt, k> - dH (log R_(i-1) + 1),
    dk += sum_(g,a2) R_(i-1) dKt; the R-step of iteration i-1 then takes dR
    back to dQhat, dk, G and dL_(i-1) as for the last one.  The first L-step
    uses the block means (R_0 uniform and constant).
    """
    Nq, d = np.shape(q)
    N = np.shape(k)[0]
    if b1 * b2 != N:
        raise ValueError(f"b1*b2 = {b1 * b2} != N = {N}")
    if Nq % b2 != 0 or Nq == 0:
        raise ValueError(f"query count {Nq} is not a positive multiple of b2 = {b2}")
    if iters < 1:
        raise ValueError("iters must be >= 1")
    b1q = Nq // b2
    bounds = tile_bounds(b1q, tiles)
    t = tiles
    s = 1.0 / math.sqrt(d)
    qb, kb, vb = _blocks(q, b1q, b2), _blocks(k, b1, b2), _blocks(v, b1, b2)
    dyb = _blocks(dy, b1q, b2)

    # ---- forward, keeping every iteration's factors
    Rs = [uniform_R(b1, b2, t)]               # R_0 .. R_T
    Ls, qhats, betas = [None], [None], [None]  # index i = 1..T
    for _ in range(iters):
        L, _ = l_step(qb, kb, Rs[-1], bounds, s)
        R, q_hat, beta = r_step(qb, kb, L, bounds, s)
        Ls.append(L)
        qhats.append(q_hat)
        betas.append(beta)
        Rs.append(R)
    T = iters
    U = np.einsum("gcap,cpd->gcad", Rs[T], vb)                # [t, c1, a2, d]

    dqb = np.zeros_like(qb)
    dkb = np.zeros_like(kb)
    dvb = np.zeros_like(vb)
    q_perm = qb.transpose(1, 0, 2)                            # [a2, a1, d]

    # gradient of the last L (through the apply) and of the last R (through U)
    dL = np.zeros_like(Ls[T])                                 # [a2, a1, c1]
    dR = np.zeros_like(Rs[T])                                 # [t, c1, a2, c2]
    for g in range(t):
        lo, hi = bounds[g], bounds[g + 1]
        Lg = Ls[T][:, lo:hi, :]                               # [a2, a1 in g, c1]
        dy_cols = dyb[lo:hi].transpose(1, 0, 2)               # [a2, a1, d]
        Ug = U[g].transpose(1, 0, 2)                          # [a2, c1, d]
        dL[:, lo:hi, :] = dy_cols @ Ug.transpose(0, 2, 1)     # <dy, U>
        dU = (Lg.transpose(0, 2, 1) @ dy_cols).transpose(1, 0, 2)  # [c1, a2, d]
        dR[g] = dU @ vb.transpose(0, 2, 1)                    # [c1, a2, c2]
        dvb += Rs[T][g].transpose(0, 2, 1) @ dU               # [c1, c2, d]

    for i in range(T, 0, -1):
        R, L, q_hat, beta = Rs[i], Ls[i], qhats[i], betas[i]
        # ---- R-step i: R = softmax(z), z = s <Qhat, k>; Qhat = sum L q / beta
        for g in range(t):
            lo, hi = bounds[g], bounds[g + 1]
            Lg = L[:, lo:hi, :]
            q_cols = q_perm[:, lo:hi, :]
            dz = R[g] * (dR[g] - np.sum(R[g] * dR[g], axis=-1, keepdims=True))
            dq_hat = s * (dz @ kb)                            # [c1, a2, d]
            dkb += s * (dz.transpose(0, 2, 1) @ q_hat[g])     # [c1, c2, d]
            mass = beta[g]                                    # [c1, a2]
            Gg = np.where((mass > 0)[:, :, None], dq_hat / np.where(mass > 0, mass, 1.0)[:, :, None], 0.0)
            Gc = Gg.transpose(1, 0, 2)                        # [a2, c1, d]
            qh_c = q_hat[g].transpose(1, 0, 2)                # [a2, c1, d]
            dL[:, lo:hi, :] += q_cols @ Gc.transpose(0, 2, 1) \
                - np.sum(Gc * qh_c, axis=-1)[:, None, :]
            dqb[lo:hi] += (Lg @ Gc).transpose(1, 0, 2)
        # ---- L-step i: L = softmax(l), l = s <q, Kt_(i-1)> + H_(i-1)
        dl = L * (dL - np.sum(L * dL, axis=-1, keepdims=True))  # [a2, a1, c1]
        Rp = Rs[i - 1]
        k_til = np.einsum("gcap,cpd->gcad", Rp, kb)           # [t, c1, a2, d]
        dk_til = np.zeros_like(k_til)
        dh = np.zeros(Rp.shape[:3])                           # [t, c1, a2]
        for g in range(t):
            lo, hi = bounds[g], bounds[g + 1]
            dlg = dl[:, lo:hi, :]                             # [a2, a1 in g, c1]
            k_cols = k_til[g].transpose(1, 0, 2)              # [a2, c1, d]
            dqb[lo:hi] += (s * (dlg @ k_cols)).transpose(1, 0, 2)
            dk_til[g] = (s * (dlg.transpose(0, 2, 1) @ q_perm[:, lo:hi, :])).transpose(1, 0, 2)
            dh[g] = dlg.sum(axis=1).T                         # [c1, a2]
        if i == 1:
            # Kt_0 = Kbar for every tile and column; H_0 is a constant
            dkb += dk_til.sum(axis=(0, 2))[:, None, :] / b2
        else:
            # Kt = R k and H = -sum R log R of the R-step before
            logR = np.log(Rp)
            dR = np.einsum("gcad,cpd->gcap", dk_til, kb) - dh[..., None] * (logR + 1.0)
            dkb += np.einsum("gcap,gcad->cpd", Rp, dk_til)
            dL = np.zeros_like(Ls[i - 1])
    return dqb.reshape(Nq, d), dkb.reshape(N, d), dvb.reshape(N, d)


def monarch_attention_grad(q, k, v, dy, b1: int, b2: int, tiles: int = 1, iters: int = 1):
    """q, dy [B, H, Nq, d], k, v [B, H, N, d] -> (dq, dk, dv) float64, head by head."""
    q, k = np.asarray(q), np.asarray(k)
    B, H, Nq, d = q.shape
    N = k.shape[2]
    out = [np.empty((B, H, Nq, d)), np.empty((B, H, N, d)), np.empty((B, H, N, d))]
    for b in range(B):
        for h in range(H):
            grads = monarch_head_grad(q[b, h], k[b, h], v[b, h], dy[b, h], b1, b2, tiles, iters)
            for o, gr in zip(out, grads):
                o[b, h] = gr
    return tuple(out)
