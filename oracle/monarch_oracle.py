"""CPU oracle for the (tiled) MonarchAttention forward pass, in float64 numpy.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or call this module.  The GPU library never does, and
this module imports nothing from the GPU package.

Sources (the web pages on MonarchRT; no code, formula or worked example is
printed there, so each step below is written from the described method):

* Monarch structure.  A fixed reshape-transpose permutation P exposes
  block-rank-1 structure, and the matrix is a product of two block-diagonal
  factors, M = P^T L P R (yunpan.plus MonarchRT article, section "Monarch
  matrices: a unified structured approximation tool").
* MonarchAttention.  The two factors L and R are optimised alternately,
  directly from Q and K, and give a dense but Monarch-structured attention
  matrix (same section, Fig. 3; VMonarch abstract: "alternating
  minimization" with an entropy term computed inside the attention kernel).
* Block alignment.  Blocks (b1, b2) = (f*h, w) for a video of N = f*h*w
  tokens: one block spans all frames and rows of one column, and blocks only
  interact along the width (yunpan.plus article, "Innovation 1: block
  alignment", Fig. 7; atlas.scime.ai summary, "Approach").
* Tiled Monarch.  Each aligned block is split into tiles, each factorised on
  its own (yunpan.plus article, "Innovation 2: tiled Monarch
  parameterisation", Fig. 2 bottom).
* Iterations.  About ten refinement iterations without finetuning, one after
  it (yunpan.plus article, "Innovation 3: finetuning and efficient kernels",
  Fig. 4 right).

Readings fixed here (the pages leave them open):

* Index convention.  Token n = a1*b2 + a2 (a1 in [b1], a2 in [b2]); key
  m = c1*b2 + c2.  L has b2 blocks of b1 x b1 (L[a2][a1, c1]); R has b1 blocks
  of b2 x b2 per tile (R[g][c1][a2, c2]).  M[(a1,a2),(c1,c2)] =
  L[a2][a1,c1] * R[g(a1)][c1][a2,c2].
* Updates.  Block coordinate ascent on the entropy-regularised objective
  F(M) = sum_n <M_n, s*S_n> + H(M_n) with S = Q K^T and s = 1/sqrt(d) (the
  variational form of softmax).  With row-stochastic factors the row entropy
  splits as H(M_n) = H(L_n) + sum_c1 L_n[c1] H(R_c1,a2), so each factor's exact
  maximiser is a block softmax:
    L-step: logits s*<q_n, Ktil[g,c1,a2]> + H(R[g,c1,a2,:]),
            Ktil[g,c1,a2] = sum_c2 R[g,c1,a2,c2] k_(c1,c2);
    R-step: logits s*<Qhat[g,c1,a2], k_(c1,c2)>,
            Qhat[g,c1,a2] = sum_(a1 in g) L[a2][a1,c1] q_(a1,a2) / beta,
            beta = sum_(a1 in g) L[a2][a1,c1].
  Where a whole tile column of L is exactly zero (beta == 0, every weight
  underflowed), Qhat := 0, so that R row is uniform.  In the last R-step that
  row only meets zero weights of L and the output does not depend on it; with
  more iterations it hands the next L-step the block mean of the keys and the
  entropy log(b2), which do enter that tile's logits.
* Start from uniform R (1/b2); one iteration = L-step then R-step; the apply
  uses the last L and R.  ``iters`` counts iterations.
* Tiles split the a1 (frame*row) index into t contiguous ranges with bounds
  floor(g*b1/t); each tile has its own R; 1 <= t <= b1.
* Natural logarithm, entropy coefficient 1, 0*log(0) = 0.
* Chunked queries against cached keys (the autoregressive, KV-cached use of
  the layer: a chunk of frames attends to the cache plus itself; yunpan.plus
  article, section on why real-time generation is hard: autoregressive,
  frame-by-frame generation with few steps).  The queries then span fewer
  blocks than the keys: queries (a1, a2) with a1 in [b1q], keys (c1, c2) with
  c1 in [b1k], the same b2.  Every formula above holds with a1 ranging over
  b1q and c1 over b1k; tiles split the query index a1.  For b1q = b1k this is
  the square layer.

Parity unpinned: whether these readings match the MonarchRT authors' own
kernels (initialisation, order, the beta temperature, the entropy term); the
pages print no formula, intermediate or output value to pin them to.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "tile_bounds", "tile_of_rows", "softmax", "entropy", "uniform_R",
    "l_step", "r_step", "apply_factors", "monarch_head", "monarch_head_adaptive",
    "dense_monarch_matrix", "explicit_monarch_matrix", "permutation_matrix",
    "objective", "row_kl",
]


# ----------------------------------------------------------------- helpers --

def tile_bounds(b1: int, t: int) -> list[int]:
    """Bounds of the t contiguous tiles of the a1 index: floor(g*b1/t)."""
    if not 1 <= t <= b1:
        raise ValueError(f"tiles must be in [1, b1]; got t={t}, b1={b1}")
    return [(g * b1) // t for g in range(t + 1)]


def tile_of_rows(b1: int, t: int) -> np.ndarray:
    """g(a1) for every a1."""
    bounds = tile_bounds(b1, t)
    g = np.empty(b1, dtype=np.int64)
    for i in range(t):
        g[bounds[i]:bounds[i + 1]] = i
    return g


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def entropy(p: np.ndarray, axis: int = -1) -> np.ndarray:
    """Shannon entropy in nats with 0*log(0) = 0."""
    plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    return -np.sum(plogp, axis=axis)


def _blocks(x: np.ndarray, b1: int, b2: int) -> np.ndarray:
    """[N, d] -> [b1, b2, d]: token a1*b2 + a2 at [a1, a2]."""
    return np.asarray(x, dtype=np.float64).reshape(b1, b2, -1)


def uniform_R(b1: int, b2: int, t: int) -> np.ndarray:
    """Starting R: every block row uniform over its b2 keys.  [t, b1, b2, b2]."""
    return np.full((t, b1, b2, b2), 1.0 / b2)


# ------------------------------------------------------------- the method --

def l_step(qb: np.ndarray, kb: np.ndarray, R: np.ndarray, bounds, s: float):
    """Exact maximiser of F over L for fixed R.

    qb: [b1q, b2, d]; kb: [b1k, b2, d]; R: [t, b1k(c1), b2(a2), b2(c2)].
    Returns L [b2(a2), b1q(a1), b1k(c1)] (rows sum to 1 over c1) and the logits.
    """
    b1q, b2, _ = qb.shape
    b1k = kb.shape[0]
    # keys aggregated through R, one per (tile, block c1, column a2)
    k_til = np.einsum("gcap,cpd->gcad", R, kb)          # [t, c1, a2, d]
    h_r = entropy(R, axis=-1)                            # [t, c1, a2]
    logits = np.empty((b2, b1q, b1k))
    for g in range(len(bounds) - 1):
        lo, hi = bounds[g], bounds[g + 1]
        q_cols = qb[lo:hi].transpose(1, 0, 2)            # [a2, a1 in g, d]
        k_cols = k_til[g].transpose(1, 0, 2)             # [a2, c1, d]
        logits[:, lo:hi, :] = s * (q_cols @ k_cols.transpose(0, 2, 1)) \
            + h_r[g].T[:, None, :]
    return softmax(logits, axis=-1), logits


def r_step(qb: np.ndarray, kb: np.ndarray, L: np.ndarray, bounds, s: float):
    """Exact maximiser of F over R for fixed L.

    L: [b2(a2), b1q(a1), b1k(c1)].  Returns R [t, c1, a2, c2], the aggregated
    queries Qhat [t, c1, a2, d] and the column masses beta [t, c1, a2].
    """
    _, b2, d = qb.shape
    b1k = kb.shape[0]
    t = len(bounds) - 1
    R = np.empty((t, b1k, b2, b2))
    q_hat = np.zeros((t, b1k, b2, d))
    beta = np.empty((t, b1k, b2))
    for g in range(t):
        lo, hi = bounds[g], bounds[g + 1]
        Lg = L[:, lo:hi, :]                               # [a2, a1 in g, c1]
        q_cols = qb[lo:hi].transpose(1, 0, 2)             # [a2, a1 in g, d]
        mass = Lg.sum(axis=1)                             # [a2, c1]
        q_til = Lg.transpose(0, 2, 1) @ q_cols            # [a2, c1, d]
        safe = np.where(mass > 0, mass, 1.0)
        qh = np.where((mass > 0)[:, :, None], q_til / safe[:, :, None], 0.0)
        q_hat[g] = qh.transpose(1, 0, 2)                  # [c1, a2, d]
        beta[g] = mass.T
        logits = s * (q_hat[g] @ kb.transpose(0, 2, 1))   # [c1, a2, c2]
        R[g] = softmax(logits, axis=-1)
    return R, q_hat, beta


def apply_factors(L: np.ndarray, R: np.ndarray, vb: np.ndarray, bounds) -> np.ndarray:
    """Y = M V without forming M: U = R V per block, then L on the permuted index.

    Returns y [b1q, b2, d] (token a1*b2 + a2 at [a1, a2]), b1q = L.shape[1].
    """
    _, b2, d = vb.shape
    y = np.empty((L.shape[1], b2, d))
    for g in range(len(bounds) - 1):
        lo, hi = bounds[g], bounds[g + 1]
        U = R[g] @ vb                                     # [c1, a2, d]
        y_cols = L[:, lo:hi, :] @ U.transpose(1, 0, 2)    # [a2, a1 in g, d]
        y[lo:hi] = y_cols.transpose(1, 0, 2)
    return y


def monarch_head(q, k, v, b1: int, b2: int, tiles: int = 1, iters: int = 1,
                 return_factors: bool = False):
    """One (batch, head): q [Nq, d], k, v [N, d] -> y [Nq, d] (float64).

    ``b1`` counts the key blocks (b1*b2 == N); the queries span
    b1q = Nq / b2 blocks (b1q == b1 for the square layer, fewer for a chunk
    of frames against cached keys).  Tiles split the query blocks.
    With ``return_factors`` also returns (L, R, history) where history holds
    the factors after every half-step (for the objective pins).
    """
    N, d = np.shape(k)
    Nq = np.shape(q)[0]
    if b1 * b2 != N:
        raise ValueError(f"b1*b2 = {b1 * b2} != N = {N}")
    if Nq % b2 != 0 or Nq == 0:
        raise ValueError(f"query count {Nq} is not a positive multiple of b2 = {b2}")
    if iters < 1:
        raise ValueError("iters must be >= 1")
    b1q = Nq // b2
    bounds = tile_bounds(b1q, tiles)
    s = 1.0 / math.sqrt(d)
    qb, kb, vb = _blocks(q, b1q, b2), _blocks(k, b1, b2), _blocks(v, b1, b2)
    R = uniform_R(b1, b2, tiles)
    history = []
    L = None
    for _ in range(iters):
        L, _ = l_step(qb, kb, R, bounds, s)
        history.append(("L", L, R))
        R, _, _ = r_step(qb, kb, L, bounds, s)
        history.append(("R", L, R))
    y = apply_factors(L, R, vb, bounds).reshape(Nq, d)
    if return_factors:
        return y, (L, R, history)
    return y


def monarch_head_adaptive(q, k, v, b1: int, b2: int, tiles: int, max_iters: int, tol: float):
    """Iterate until the objective stops improving (training-free regime).

    The pages run about ten iterations without finetuning (yunpan.plus
    article, "Innovation 3", Fig. 4 right) and give no stopping rule.  Reading
    used here: after the L-step of iteration i the factors (L_i, R_(i-1))
    have objective F_i = sum_n logsumexp of that L-step's logits (L_i is the
    exact maximiser for R_(i-1)); stop after iteration i when i == max_iters,
    or when i >= 2 and (F_i - F_(i-1)) / Nq <= tol (gain per query token, in
    nats).  Iteration i's R-step is then the last and the apply uses L_i, R_i.
    Returns (y, iterations used, [F_1, F_2, ...]).
    """
    N, d = np.shape(k)
    Nq = np.shape(q)[0]
    if b1 * b2 != N or Nq % b2 != 0 or Nq == 0:
        raise ValueError("bad block sizes")
    if max_iters < 1:
        raise ValueError("max_iters must be >= 1")
    b1q = Nq // b2
    tb = tile_bounds(b1q, tiles)
    s = 1.0 / math.sqrt(d)
    qb, kb, vb = _blocks(q, b1q, b2), _blocks(k, b1, b2), _blocks(v, b1, b2)
    R = uniform_R(b1, b2, tiles)
    F = []
    it = 0
    while True:
        it += 1
        L, logits = l_step(qb, kb, R, tb, s)
        m = np.max(logits, axis=-1, keepdims=True)
        F.append(float(np.sum(m[..., 0] + np.log(np.sum(np.exp(logits - m), axis=-1)))))
        R, _, _ = r_step(qb, kb, L, tb, s)
        if it >= max_iters or (it >= 2 and (F[-1] - F[-2]) / Nq <= tol):
            break
    out = apply_factors(L, R, vb, tb).reshape(Nq, d)
    return out, it, F


# ----------------------------------------------- dense forms and objective --

def dense_monarch_matrix(L: np.ndarray, R: np.ndarray, bounds) -> np.ndarray:
    """M[(a1,a2),(c1,c2)] = L[a2][a1,c1] * R[g(a1)][c1][a2,c2], as [Nq, N]."""
    b2, b1q, b1k = L.shape
    g_of = tile_of_rows(b1q, len(bounds) - 1)
    M = np.empty((b1q, b2, b1k, b2))
    for a1 in range(b1q):
        Rg = R[g_of[a1]]                                  # [c1, a2, c2]
        # M[a1, a2, c1, c2] = L[a2, a1, c1] * Rg[c1, a2, c2]
        M[a1] = L[:, a1, :][:, :, None] * Rg.transpose(1, 0, 2)
    return M.reshape(b1q * b2, b1k * b2)


def permutation_matrix(b1: int, b2: int) -> np.ndarray:
    """P with P e_(a1*b2+a2) = e_(a2*b1+a1): the reshape-transpose permutation."""
    N = b1 * b2
    P = np.zeros((N, N))
    for a1 in range(b1):
        for a2 in range(b2):
            P[a2 * b1 + a1, a1 * b2 + a2] = 1.0
    return P


def explicit_monarch_matrix(L: np.ndarray, R0: np.ndarray) -> np.ndarray:
    """Plain (one-tile) Monarch written as a matrix product P^T L P R.

    L: [b2, b1, b1] blocks (block a2 acts on the a2-th group of b1 entries
    after P); R0: [b1(c1), b2(a2), b2(c2)] blocks.  In the (c1,c2) key basis
    R is block diagonal with blocks indexed by c1, whose (a2, c2) entry is
    R0[c1, a2, c2]; in the permuted basis L is block diagonal with blocks
    indexed by a2.
    """
    b2, b1, _ = L.shape
    N = b1 * b2
    P = permutation_matrix(b1, b2)
    Lbd = np.zeros((N, N))
    for a2 in range(b2):
        Lbd[a2 * b1:(a2 + 1) * b1, a2 * b1:(a2 + 1) * b1] = L[a2]
    Rbd = np.zeros((N, N))
    for c1 in range(b1):
        Rbd[c1 * b2:(c1 + 1) * b2, c1 * b2:(c1 + 1) * b2] = R0[c1]
    return P.T @ Lbd @ P @ Rbd


def objective(M: np.ndarray, q, k) -> float:
    """F(M) = sum_n <M_n, s*S_n> + H(M_n) with S = Q K^T, s = 1/sqrt(d)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = 1.0 / math.sqrt(q.shape[-1])
    return float(np.sum(M * (s * (q @ k.T))) + np.sum(entropy(M, axis=-1)))


def row_kl(M: np.ndarray, A: np.ndarray) -> np.ndarray:
    """KL(M_n || A_n) for every row n (A strictly positive)."""
    ratio = np.where(M > 0, M / A, 1.0)
    return np.sum(np.where(M > 0, M * np.log(ratio), 0.0), axis=-1)
