"""Checks that pin the CPU oracle to facts outside itself.

Each ``check_*`` takes an oracle module (the real one, or a copy with a
planted mistake) and raises AssertionError when the fact does not hold.  The
facts come from the mathematics of the method and from textbook attention,
never from the oracle's own output:

* row-stochastic attention rows, and the factored apply equal to the dense
  Monarch matrix times V;
* the one-tile case equal to the plain Monarch product P^T L P R written out
  with an explicit permutation matrix;
* degenerate block shapes and one-row tiles reduce to dense softmax attention
  (computed by torch's scaled_dot_product_attention in float64);
* Q = 0 gives the uniform matrix (every output row is the mean of V);
* every half-step is the exact maximiser of the entropy-regularised objective
  (checked by numerical optimisation with scipy), so the objective never
  decreases, and the objective equals sum lse - sum KL to dense attention;
* block rank at most the tile count, and the KKT (log-softmax) conditions;
* an exactly separable positional input is reproduced exactly by aligned
  blocks in one iteration, and an input separable into frame and position
  parts by blocks of whole frames;
* chunked queries against cached keys: row-stochastic non-square M equal to
  the factored apply, exact attention where the blocks degenerate, and a chunk
  equal to the matching rows of the square layer over all frames.
"""
from __future__ import annotations

import math

import numpy as np

TOL = 1e-10


def _rand(rng, *shape, scale=1.0):
    return scale * rng.standard_normal(shape)


def _sdpa(q, k, v):
    """Dense softmax attention from torch (library routine), float64 on CPU."""
    import torch
    import torch.nn.functional as F
    tq = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, None]
    tk = torch.from_numpy(np.asarray(k, dtype=np.float64))[None, None]
    tv = torch.from_numpy(np.asarray(v, dtype=np.float64))[None, None]
    return F.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()


def _dense_A(q, k):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    x = (q @ k.T) / math.sqrt(q.shape[1])
    x = x - x.max(axis=1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=1, keepdims=True)


def _case(seed=0, b1=6, b2=5, d=8, scale=1.5):
    rng = np.random.default_rng(seed)
    N = b1 * b2
    return (_rand(rng, N, d, scale=scale), _rand(rng, N, d, scale=scale),
            _rand(rng, N, d))


# ----------------------------------------------------------------- checks --

def check_tile_bounds(orc):
    for b1 in (1, 2, 7, 90, 630, 945):
        for t in (1, 2, 3, 4, 8):
            if t > b1:
                continue
            bd = orc.tile_bounds(b1, t)
            assert bd[0] == 0 and bd[-1] == b1 and len(bd) == t + 1
            sizes = np.diff(bd)
            assert sizes.min() >= 1 and sizes.max() - sizes.min() <= 1
            if 2 * t <= b1:
                assert set(bd) <= set(orc.tile_bounds(b1, 2 * t))
            g = orc.tile_of_rows(b1, t)
            assert np.all(np.diff(g) >= 0) and g[0] == 0 and g[-1] == t - 1


def check_row_stochastic_and_dense_apply(orc):
    """O1 + O2: M >= 0, rows sum to one, factored apply == M @ V."""
    for (b1, b2, t, T) in [(6, 5, 1, 1), (6, 5, 2, 2), (5, 6, 3, 1), (4, 4, 4, 2)]:
        q, k, v = _case(1, b1, b2)
        y, (L, R, _) = orc.monarch_head(q, k, v, b1, b2, t, T, return_factors=True)
        M = orc.dense_monarch_matrix(L, R, orc.tile_bounds(b1, t))
        assert M.min() >= 0.0
        assert np.max(np.abs(M.sum(axis=1) - 1.0)) <= 1e-12
        assert np.max(np.abs(M @ v - y)) <= 1e-12


def check_plain_monarch_product(orc):
    """O3 + O12: one tile equals P^T L P R with an explicit permutation."""
    b1, b2 = 5, 3
    P = orc.permutation_matrix(b1, b2)
    assert np.array_equal(P @ P.T, np.eye(b1 * b2))
    # P is the (b1,b2) -> (b2,b1) transpose of a row-major index grid
    x = np.arange(b1 * b2, dtype=np.float64)
    assert np.array_equal(P @ x, x.reshape(b1, b2).T.ravel())
    for T in (1, 2):
        q, k, v = _case(2, b1, b2)
        y, (L, R, _) = orc.monarch_head(q, k, v, b1, b2, 1, T, return_factors=True)
        M_plain = orc.explicit_monarch_matrix(L, R[0])
        M = orc.dense_monarch_matrix(L, R, [0, b1])
        assert np.max(np.abs(M - M_plain)) <= 1e-14
        assert np.max(np.abs(M_plain @ v - y)) <= 1e-12


def check_degenerate_blocks_are_dense_attention(orc):
    """O4: (b1,b2) = (1,N) or (N,1) is exactly softmax attention."""
    q, k, v = _case(3, 4, 6)
    N = q.shape[0]
    ref = _sdpa(q, k, v)
    for (b1, b2) in [(1, N), (N, 1)]:
        for T in (1, 2):
            y = orc.monarch_head(q, k, v, b1, b2, 1, T)
            assert np.max(np.abs(y - ref)) <= TOL, (b1, b2, T)


def check_one_row_tiles(orc):
    """O4: t = b1.  T >= 2 is exact dense attention; T = 1 has a closed form:
    L = softmax over blocks of s*q.kbar_c1 (kbar = block mean of keys),
    R = softmax within the block of s*q.k."""
    b1, b2, d = 5, 4, 8
    q, k, v = _case(4, b1, b2, d)
    ref = _sdpa(q, k, v)
    for T in (2, 3):
        y = orc.monarch_head(q, k, v, b1, b2, b1, T)
        assert np.max(np.abs(y - ref)) <= TOL, T
    y1 = orc.monarch_head(q, k, v, b1, b2, b1, 1)
    s = 1.0 / math.sqrt(d)
    kb = k.reshape(b1, b2, d)
    kbar = kb.mean(axis=1)
    expect = np.empty_like(v)
    vb = v.reshape(b1, b2, d)
    for n in range(b1 * b2):
        lw = np.exp(s * (kbar @ q[n]))
        lw /= lw.sum()
        acc = np.zeros(d)
        for c1 in range(b1):
            rw = np.exp(s * (kb[c1] @ q[n]))
            rw /= rw.sum()
            acc += lw[c1] * (rw @ vb[c1])
        expect[n] = acc
    assert np.max(np.abs(y1 - expect)) <= TOL


def _sdpa_masked(q, k, v, keep):
    """torch's dense attention in float64 over the keys where ``keep``."""
    import torch
    import torch.nn.functional as F
    mask = torch.where(torch.from_numpy(np.asarray(keep)), 0.0, -math.inf).to(torch.float64)
    tq, tk, tv = (torch.from_numpy(np.asarray(x, dtype=np.float64))[None, None] for x in (q, k, v))
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask[None, :])[0, 0].numpy()


def check_beta_zero_branch(orc):
    """A key block whose weight underflows to exactly 0 in every tile column
    (beta = 0, reading D6: that R row is uniform, i.e. Qhat := 0).

    The block mean of block c* lies about 892 nats below every other block
    for every query, so the first L-step gives it weight 0 exactly; its key 0
    is every query's best single match.  Under the reading the uniform R row
    hands the next L-step the block mean again (plus log b2), so the block
    keeps weight 0 and can be deleted:
      * one-row tiles, T = 2, 3: exact softmax attention over the keys outside
        block c* (torch SDPA with a mask; t = b1 with T >= 2 is exact attention
        over blocks that keep their weight);
      * two tiles, T = 2: the same layer with block c* removed from the keys
        (queries over 8 blocks, keys over 7).
    Any other choice for Qhat (a tile mean of q, say) gives the block its
    best key in the second L-step and a weight near 1."""
    from structured_attention_video_monarch_amd.inputs import make_underflow_head
    b1, b2, d, cstar = 8, 4, 16, 3
    q, k, v = (x.astype(np.float64) for x in make_underflow_head(0, b1, b2, d, cstar))
    keep = np.ones(b1 * b2, dtype=bool)
    keep[cstar * b2:(cstar + 1) * b2] = False
    # the branch is reached: the first L-step's weights on block c* are 0
    _, (_, _, hist) = orc.monarch_head(q, k, v, b1, b2, b1, 2, return_factors=True)
    assert np.all(hist[0][1][:, :, cstar] == 0.0)
    ref = _sdpa_masked(q, k, v, keep)
    for T in (2, 3):
        y = orc.monarch_head(q, k, v, b1, b2, b1, T)
        assert np.max(np.abs(y - ref)) <= TOL, T
    y2 = orc.monarch_head(q, k, v, b1, b2, 2, 2)
    y2_del = orc.monarch_head(q, k[keep], v[keep], b1 - 1, b2, 2, 2)
    assert np.max(np.abs(y2 - y2_del)) <= 1e-12


def check_zero_queries_uniform(orc):
    """O5: Q = 0 makes every logit equal, so M = 1/N and y_n = mean(V)."""
    b1, b2, d = 6, 4, 8
    _, k, v = _case(5, b1, b2, d)
    q = np.zeros_like(k)
    for t in (1, 3):
        y = orc.monarch_head(q, k, v, b1, b2, t, 2)
        assert np.max(np.abs(y - v.mean(axis=0))) <= 1e-12


def check_objective_ascent_and_identity(orc):
    """O6: F never decreases over the 2T half-steps, and
    F(M) = sum_n logsumexp(s S_n) - sum_n KL(M_n || A_n)."""
    b1, b2, d = 6, 5, 8
    q, k, v = _case(6, b1, b2, d, scale=2.0)
    s = 1.0 / math.sqrt(d)
    A = _dense_A(q, k)
    S = s * (q @ k.T)
    lse = np.log(np.sum(np.exp(S - S.max(axis=1, keepdims=True)), axis=1)) + S.max(axis=1)
    for t in (1, 2, 3):
        bounds = orc.tile_bounds(b1, t)
        _, (_, _, hist) = orc.monarch_head(q, k, v, b1, b2, t, 3, return_factors=True)
        prev = -np.inf
        for _, L, R in hist:
            M = orc.dense_monarch_matrix(L, R, bounds)
            F = orc.objective(M, q, k)
            # independent evaluation of F for the identity
            ent = -np.sum(np.where(M > 0, M * np.log(np.where(M > 0, M, 1)), 0))
            F_direct = float(np.sum(M * S) + ent)
            assert abs(F - F_direct) <= 1e-9 * max(1.0, abs(F))
            kl = orc.row_kl(M, A)
            assert np.all(kl >= -1e-12)
            assert abs(F - (lse.sum() - kl.sum())) <= 1e-9 * max(1.0, abs(F))
            assert F >= prev - 1e-10, (t, F, prev)
            prev = F


def check_steps_are_exact_maximisers(orc):
    """Each half-step maximises F over its factor: compare the closed form with
    a generic numerical maximisation (scipy L-BFGS over free logits)."""
    from scipy.optimize import minimize
    b1, b2, d = 3, 2, 4
    N = b1 * b2
    q, k, _ = _case(7, b1, b2, d)
    s = 1.0 / math.sqrt(d)
    S = s * (q @ k.T)
    rng = np.random.default_rng(0)
    t = 1
    bounds = [0, b1]
    R = orc.softmax(rng.standard_normal((t, b1, b2, b2)), axis=-1)
    qb, kb = q.reshape(b1, b2, d), k.reshape(b1, b2, d)

    def F_of(L, Rf):
        M = np.empty((b1, b2, b1, b2))
        for a1 in range(b1):
            for a2 in range(b2):
                for c1 in range(b1):
                    M[a1, a2, c1] = L[a2, a1, c1] * Rf[0, c1, a2]
        M = M.reshape(N, N)
        ent = -np.sum(np.where(M > 0, M * np.log(np.where(M > 0, M, 1)), 0))
        return float(np.sum(M * S) + ent)

    def sm(z, shape):
        z = z.reshape(shape)
        z = z - z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=-1, keepdims=True)

    L_closed, _ = orc.l_step(qb, kb, R, bounds, s)
    res = minimize(lambda z: -F_of(sm(z, (b2, b1, b1)), R), np.zeros(b2 * b1 * b1),
                   method="L-BFGS-B", options={"gtol": 1e-12, "ftol": 1e-15, "maxiter": 5000})
    L_num = sm(res.x, (b2, b1, b1))
    assert np.max(np.abs(L_num - L_closed)) <= 2e-5
    assert F_of(L_closed, R) >= -res.fun - 1e-9

    R_closed, _, _ = orc.r_step(qb, kb, L_closed, bounds, s)
    res = minimize(lambda z: -F_of(L_closed, sm(z, (t, b1, b2, b2))), np.zeros(t * b1 * b2 * b2),
                   method="L-BFGS-B", options={"gtol": 1e-12, "ftol": 1e-15, "maxiter": 5000})
    R_num = sm(res.x, (t, b1, b2, b2))
    assert np.max(np.abs(R_num - R_closed)) <= 2e-5
    assert F_of(L_closed, R_closed) >= -res.fun - 1e-9


def check_block_rank_at_most_tiles(orc):
    """O7: block (a2, c1) of P M P^T has rank <= t; one tile's rows, rank 1."""
    b1, b2, d = 8, 4, 8
    q, k, v = _case(8, b1, b2, d)
    for t in (1, 2, 4):
        bounds = orc.tile_bounds(b1, t)
        _, (L, R, _) = orc.monarch_head(q, k, v, b1, b2, t, 2, return_factors=True)
        M = orc.dense_monarch_matrix(L, R, bounds).reshape(b1, b2, b1, b2)
        for a2 in range(b2):
            for c1 in range(b1):
                blk = M[:, a2, c1, :]                     # rows a1, cols c2
                sv = np.linalg.svd(blk, compute_uv=False)
                assert np.sum(sv > 1e-12 * sv[0]) <= t
                for g in range(t):
                    sub = np.linalg.svd(blk[bounds[g]:bounds[g + 1]], compute_uv=False)
                    assert np.sum(sub > 1e-12 * max(sub[0], 1e-300)) <= 1


def check_kkt(orc):
    """O11: log L - logits is constant along each L row; same for R."""
    b1, b2, d = 6, 5, 8
    q, k, _ = _case(9, b1, b2, d)
    s = 1.0 / math.sqrt(d)
    qb, kb = q.reshape(b1, b2, d), k.reshape(b1, b2, d)
    bounds = orc.tile_bounds(b1, 2)
    R = orc.uniform_R(b1, b2, 2)
    for _ in range(2):
        L, logits = orc.l_step(qb, kb, R, bounds, s)
        gap = np.log(L) - logits
        assert np.max(np.abs(gap - gap[..., :1])) <= 1e-12
        assert np.max(np.abs(L.sum(-1) - 1)) <= 1e-12
        R, q_hat, beta = orc.r_step(qb, kb, L, bounds, s)
        rl = s * np.einsum("gcad,cpd->gcap", q_hat, kb)
        gap = np.log(R) - rl
        assert np.max(np.abs(gap - gap[..., :1])) <= 1e-12
        # the aggregated query is the L-weighted mean of the tile's queries
        g, c1, a2 = 1, 2, 3
        lo, hi = bounds[g], bounds[g + 1]
        w = L[a2, lo:hi, c1]
        assert abs(beta[g, c1, a2] - w.sum()) <= 1e-14
        assert np.max(np.abs(q_hat[g, c1, a2] - (w @ qb[lo:hi, a2]) / w.sum())) <= 1e-12


def check_separable_positional_exact(orc):
    """O8: logits that split into a (frame,row) part plus a column part are
    reproduced exactly by aligned blocks in one iteration; a token shuffle
    breaks it."""
    from structured_attention_video_monarch_amd.inputs import positional_term
    f, h, w, d = 2, 3, 4, 24
    pos = positional_term(f, h, w, d, 1.0)
    q = k = pos
    rng = np.random.default_rng(10)
    v = rng.standard_normal(pos.shape)
    b1, b2 = f * h, w
    dense = _sdpa(q, k, v)
    y, (L, R, _) = orc.monarch_head(q, k, v, b1, b2, 1, 1, return_factors=True)
    assert np.max(np.abs(y - dense)) <= 1e-10
    M = orc.dense_monarch_matrix(L, R, [0, b1])
    assert np.max(np.abs(orc.row_kl(M, _dense_A(q, k)))) <= 1e-10
    perm = rng.permutation(q.shape[0])
    qs, ks = q[perm], k[perm]
    _, (L, R, _) = orc.monarch_head(qs, ks, v[perm], b1, b2, 1, 1, return_factors=True)
    Ms = orc.dense_monarch_matrix(L, R, [0, b1])
    assert orc.row_kl(Ms, _dense_A(qs, ks)).mean() >= 1e-4


def check_frame_separable_exact(orc):
    """Blocks of whole frames, (b1, b2) = (f, h*w) (reading D15): logits that
    split into a part depending on the two frames plus a part depending on
    the two positions within a frame make attention the product of a frame
    softmax and a position softmax, which these blocks reproduce exactly in
    one iteration for any tile count; blocks of half frames do not."""
    f, hw, d1, d2 = 4, 6, 5, 7
    rng = np.random.default_rng(11)
    qf, kf = rng.standard_normal((f, d1)), rng.standard_normal((f, d1))
    qp, kp = rng.standard_normal((hw, d2)), rng.standard_normal((hw, d2))
    # token n = frame * hw + position; features [frame part, position part]
    q = 1.3 * np.concatenate([np.repeat(qf, hw, axis=0), np.tile(qp, (f, 1))], axis=1)
    k = 1.3 * np.concatenate([np.repeat(kf, hw, axis=0), np.tile(kp, (f, 1))], axis=1)
    v = rng.standard_normal((f * hw, d1 + d2))
    dense = _sdpa(q, k, v)
    for t in (1, 2, 4):
        y = orc.monarch_head(q, k, v, f, hw, t, 1)
        assert np.max(np.abs(y - dense)) <= TOL, t
    y = orc.monarch_head(q, k, v, 2 * f, hw // 2, 1, 1)
    assert np.max(np.abs(y - dense)) >= 1e-4


# --------------------------------------- chunked queries, cached keys (KV) --

def check_kv_row_stochastic_and_dense_apply(orc):
    """Chunk of query blocks against more key blocks: M is [Nq, N] row-stochastic
    and the factored apply equals the dense product."""
    rng = np.random.default_rng(50)
    for (b1q, b1k, b2, t, T) in [(4, 10, 3, 1, 1), (4, 10, 3, 2, 2), (3, 7, 5, 3, 1)]:
        q = 1.5 * rng.standard_normal((b1q * b2, 8))
        k = 1.5 * rng.standard_normal((b1k * b2, 8))
        v = rng.standard_normal((b1k * b2, 8))
        y, (L, R, _) = orc.monarch_head(q, k, v, b1k, b2, t, T, return_factors=True)
        assert y.shape == (b1q * b2, 8)
        M = orc.dense_monarch_matrix(L, R, orc.tile_bounds(b1q, t))
        assert M.shape == (b1q * b2, b1k * b2)
        assert M.min() >= 0.0
        assert np.max(np.abs(M.sum(axis=1) - 1.0)) <= 1e-12
        assert np.max(np.abs(M @ v - y)) <= 1e-12


def check_kv_exact_cases(orc):
    """b2 = 1 (any tiles, iterations) and one key block with one-row tiles are
    exact softmax attention of the chunk's queries over all keys."""
    rng = np.random.default_rng(51)
    Nq, Nk, d = 12, 30, 8
    q = 1.5 * rng.standard_normal((Nq, d))
    k = 1.5 * rng.standard_normal((Nk, d))
    v = rng.standard_normal((Nk, d))
    ref = _sdpa(q, k, v)
    for t, T in [(1, 1), (4, 2), (12, 1)]:
        y = orc.monarch_head(q, k, v, Nk, 1, t, T)
        assert np.max(np.abs(y - ref)) <= TOL, ("b2=1", t, T)
    # one key block (b1k = 1, b2 = Nk): queries must come in whole blocks of b2
    q2 = 1.5 * rng.standard_normal((3 * Nk, d))
    ref2 = _sdpa(q2, k, v)
    for T in (1, 3):
        y = orc.monarch_head(q2, k, v, 1, Nk, 3, T)
        assert np.max(np.abs(y - ref2)) <= TOL, ("b1k=1", T)


def check_kv_chunk_is_last_tiles_of_full_layer(orc):
    """A chunk of the last fq frames against all fk frames equals the rows of
    the square layer over all frames whose tiles cover exactly the chunk with
    the same bounds (t_full = t * fk / fq): tiles are independent query-row
    groups, and the chunk's rows see the same keys."""
    rng = np.random.default_rng(52)
    fk, fq, h, w, d = 6, 2, 3, 4, 8
    b1k, b2 = fk * h, w
    N, Nq = b1k * b2, fq * h * w
    q = 1.5 * rng.standard_normal((N, d))
    k = 1.5 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    for t in (1, 2, 3):
        for T in (1, 2):
            full = orc.monarch_head(q, k, v, b1k, b2, t * fk // fq, T)
            chunk = orc.monarch_head(q[N - Nq:], k, v, b1k, b2, t, T)
            assert np.max(np.abs(chunk - full[N - Nq:])) <= 1e-12, (t, T)


# ------------------------------------------------ iterating to convergence --

def check_adaptive_iterations(orc):
    """Early stopping: F_i equals the dense objective of (L_i, R_(i-1)); the
    stop is the first i >= 2 whose gain per token is <= tol (computed from the
    dense objectives); never stopping early equals max_iters iterations, and
    stopping at once equals two."""
    b1, b2, t, d = 6, 5, 2, 8
    q, k, v = _case(60, b1, b2, d)
    N = b1 * b2
    # dense objectives after each L-step, from the factors of a long run
    _, (_, _, hist) = orc.monarch_head(q, k, v, b1, b2, t, 6, return_factors=True)
    bounds = orc.tile_bounds(b1, t)
    F_dense = [orc.objective(orc.dense_monarch_matrix(L, R, bounds), q, k)
               for (kind, L, R) in hist if kind == "L"]
    y, used, F = orc.monarch_head_adaptive(q, k, v, b1, b2, t, 6, -1.0)
    assert used == 6
    assert np.max(np.abs(np.array(F) - np.array(F_dense))) <= 1e-9 * max(1.0, abs(F_dense[0]))
    assert np.max(np.abs(y - orc.monarch_head(q, k, v, b1, b2, t, 6))) <= 1e-12
    gains = np.diff(F_dense) / N
    assert np.all(gains >= -1e-12)
    for tol in (1e30, float(gains[1]) * 1.0001, float(gains[2]) * 1.0001, 0.0):
        want = next((i + 2 for i, g in enumerate(gains) if g <= tol), 6)
        y, used, _ = orc.monarch_head_adaptive(q, k, v, b1, b2, t, 6, tol)
        assert used == want, (tol, used, want)
        assert np.max(np.abs(y - orc.monarch_head(q, k, v, b1, b2, t, want))) <= 1e-12
    y1, used1, _ = orc.monarch_head_adaptive(q, k, v, b1, b2, t, 1, 1e30)
    assert used1 == 1 and np.max(np.abs(y1 - orc.monarch_head(q, k, v, b1, b2, t, 1))) <= 1e-12


ALL_CHECKS = [
    check_tile_bounds,
    check_row_stochastic_and_dense_apply,
    check_plain_monarch_product,
    check_degenerate_blocks_are_dense_attention,
    check_one_row_tiles,
    check_zero_queries_uniform,
    check_beta_zero_branch,
    check_objective_ascent_and_identity,
    check_steps_are_exact_maximisers,
    check_block_rank_at_most_tiles,
    check_kkt,
    check_kv_row_stochastic_and_dense_apply,
    check_kv_exact_cases,
    check_kv_chunk_is_last_tiles_of_full_layer,
    check_adaptive_iterations,
    check_separable_positional_exact,
    check_frame_separable_exact,
]
