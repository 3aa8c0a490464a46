"""CPU oracle for the gradient of the one-iteration tiled MonarchAttention
forward (float64 numpy).

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

Pinned by central finite differences of the forward oracle and by the two
block shapes where the method is exact softmax attention (tests).  Only one
iteration: a gradient through several unrolled iterations is not covered.
"""
from __future__ import annotations

import math

import numpy as np

from .monarch_oracle import _blocks, l_step, r_step, tile_bounds, uniform_R

__all__ = ["monarch_head_grad", "monarch_attention_grad"]


def monarch_head_grad(q, k, v, dy, b1: int, b2: int, tiles: int = 1):
    """Gradient of sum(dy * y) for one (batch, head) at one iteration.

    q, k, v, dy: [N, d].  Returns (dq, dk, dv), each [N, d] float64.
    """
    N, d = np.shape(q)
    if b1 * b2 != N:
        raise ValueError(f"b1*b2 = {b1 * b2} != N = {N}")
    bounds = tile_bounds(b1, tiles)
    t = tiles
    s = 1.0 / math.sqrt(d)
    qb, kb, vb = _blocks(q, b1, b2), _blocks(k, b1, b2), _blocks(v, b1, b2)
    dyb = _blocks(dy, b1, b2)

    # ---- forward, keeping what the reverse needs
    kbar = kb.mean(axis=1)                                   # [c1, d]
    L, _ = l_step(qb, kb, uniform_R(b1, b2, t), bounds, s)  # [a2, a1, c1]
    R, q_hat, beta = r_step(qb, kb, L, bounds, s)            # [t,c1,a2,c2], [t,c1,a2,d], [t,c1,a2]
    U = np.einsum("gcap,cpd->gcad", R, vb)                   # [t, c1, a2, d]

    dqb = np.zeros_like(qb)
    dkb = np.zeros_like(kb)
    dvb = np.zeros_like(vb)
    dL = np.zeros_like(L)                                    # [a2, a1, c1]
    G = np.zeros_like(q_hat)                                 # [t, c1, a2, d]

    for g in range(t):
        lo, hi = bounds[g], bounds[g + 1]
        Lg = L[:, lo:hi, :]                                  # [a2, a1 in g, c1]
        dy_cols = dyb[lo:hi].transpose(1, 0, 2)              # [a2, a1, d]
        q_cols = qb[lo:hi].transpose(1, 0, 2)                # [a2, a1, d]
        Ug = U[g].transpose(1, 0, 2)                         # [a2, c1, d]
        # apply: y = L U
        dL[:, lo:hi, :] = dy_cols @ Ug.transpose(0, 2, 1)    # <dy, U>
        dU = (Lg.transpose(0, 2, 1) @ dy_cols).transpose(1, 0, 2)  # [c1, a2, d]
        # U = R v
        dR = dU @ vb.transpose(0, 2, 1)                      # [c1, a2, c2]
        dvb += R[g].transpose(0, 2, 1) @ dU                  # [c1, c2, d]
        # R = softmax(z)
        dz = R[g] * (dR - np.sum(R[g] * dR, axis=-1, keepdims=True))
        dq_hat = s * (dz @ kb)                               # [c1, a2, d]
        dkb += s * (dz.transpose(0, 2, 1) @ q_hat[g])        # [c1, c2, d]
        # Qhat = sum L q / beta
        mass = beta[g]                                       # [c1, a2]
        Gg = np.where((mass > 0)[:, :, None], dq_hat / np.where(mass > 0, mass, 1.0)[:, :, None], 0.0)
        G[g] = Gg
        Gc = Gg.transpose(1, 0, 2)                           # [a2, c1, d]
        qh_c = q_hat[g].transpose(1, 0, 2)                   # [a2, c1, d]
        dL[:, lo:hi, :] += q_cols @ Gc.transpose(0, 2, 1) \
            - np.sum(Gc * qh_c, axis=-1)[:, None, :]
        dqb[lo:hi] += (Lg @ Gc).transpose(1, 0, 2)

    # L = softmax(l), l = s <q, Kbar>
    dl = L * (dL - np.sum(L * dL, axis=-1, keepdims=True))  # [a2, a1, c1]
    q_perm = qb.transpose(1, 0, 2)                           # [a2, a1, d]
    dqb += (s * (dl @ kbar)).transpose(1, 0, 2)
    dkbar = s * np.einsum("pac,pad->cd", dl, q_perm)         # [c1, d]
    dkb += dkbar[:, None, :] / b2
    return dqb.reshape(N, d), dkb.reshape(N, d), dvb.reshape(N, d)


def monarch_attention_grad(q, k, v, dy, b1: int, b2: int, tiles: int = 1):
    """[B, H, N, d] inputs -> (dq, dk, dv) float64, head by head."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    out = [np.empty((B, H, N, d)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            grads = monarch_head_grad(q[b, h], k[b, h], v[b, h], dy[b, h], b1, b2, tiles)
            for o, gr in zip(out, grads):
                o[b, h] = gr
    return tuple(out)
