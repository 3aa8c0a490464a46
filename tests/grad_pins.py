"""Checks that pin the CPU gradient oracle to facts outside itself.

Each ``check_*`` takes a gradient module (``oracle.monarch_grad``, or a copy
with a planted mistake) and raises AssertionError when the fact does not hold
(one and several iterations):

* central finite differences of the forward oracle along random directions,
  for each input separately, and entry by entry on a tiny case;
* the block shapes where the method is exact softmax attention
  ((b1, b2) = (N, 1), any tiles; (1, N); one-row tiles with two or more
  iterations), against torch autograd through torch's own attention in
  float64;
* one-row tiles (t = b1), where the forward has a closed form that does not
  go through the aggregation, against torch autograd of that closed form;
* symmetries of the forward: a shift of every key leaves y unchanged (the
  key gradient sums to zero), a shift of every value shifts every output row
  (the value gradient sums to sum(dy)), and q -> a q, k -> k / a leaves y
  unchanged (<dq, q> = <dk, k>);
* a chunk of query frames against all keys: finite differences as above;
  blocks of one key (b2 = 1), exact attention of the chunk's queries over all
  keys; and the square layer over all frames whose tiles cover the chunk with
  the same bounds, with dy zero outside the chunk, has the chunk's gradient.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

REL = 1e-7


def _case(seed, b1, b2, d, scale=1.5):
    rng = np.random.default_rng(seed)
    N = b1 * b2
    q = scale * rng.standard_normal((N, d))
    k = scale * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    dy = rng.standard_normal((N, d))
    return q, k, v, dy


def _loss(q, k, v, dy, b1, b2, t, T=1):
    return float(np.sum(dy * oracle.monarch_head(q, k, v, b1, b2, t, T)))


def _torch_grads(fn, q, k, v, dy):
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    y = fn(tq, tk, tv)
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _close(a, b, rel, what):
    err = np.max(np.abs(a - b))
    scale = max(np.max(np.abs(b)), 1e-300)
    assert err <= rel * scale, f"{what}: max err {err:.3e} vs scale {scale:.3e}"


# ----------------------------------------------------------------- checks --

def check_grad_directional_fd(grd):
    """d/dh sum(dy * y(x + h u)) at h = 0 equals <grad, u>, per input."""
    h = 1e-5
    for seed, (b1, b2, t, d, T) in enumerate([(6, 4, 1, 8, 1), (6, 4, 2, 8, 1), (5, 6, 3, 4, 1), (7, 3, 7, 4, 1),
                                              (8, 5, 4, 16, 1), (6, 4, 1, 8, 2), (6, 4, 2, 8, 3),
                                              (5, 6, 3, 4, 2), (8, 5, 4, 16, 3)]):
        q, k, v, dy = _case(seed, b1, b2, d)
        dq, dk, dv = grd.monarch_head_grad(q, k, v, dy, b1, b2, t, T)
        rng = np.random.default_rng(100 + seed)
        for which, g in (("q", dq), ("k", dk), ("v", dv)):
            u = rng.standard_normal(q.shape)
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[which] = args_p[which] + h * u
            args_m[which] = args_m[which] - h * u
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], dy, b1, b2, t, T)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], dy, b1, b2, t, T)) / (2 * h)
            an = float(np.sum(g * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                f"{which} ({b1},{b2},t={t},T={T}): fd {fd:.10f} vs analytic {an:.10f}"


def check_grad_entrywise_fd(grd):
    """Every entry of dq, dk, dv by central differences on a tiny case."""
    b1, b2, t, d = 3, 2, 2, 3
    q, k, v, dy = _case(7, b1, b2, d)
    h = 1e-5
    for T in (1, 2):
        grads = grd.monarch_head_grad(q, k, v, dy, b1, b2, t, T)
        for idx, (name, g) in enumerate(zip("qkv", grads)):
            base = [q, k, v]
            fd = np.empty_like(g)
            for i in range(g.shape[0]):
                for j in range(g.shape[1]):
                    xp = [x.copy() for x in base]
                    xm = [x.copy() for x in base]
                    xp[idx][i, j] += h
                    xm[idx][i, j] -= h
                    fd[i, j] = (_loss(*xp, dy, b1, b2, t, T) - _loss(*xm, dy, b1, b2, t, T)) / (2 * h)
            _close(g, fd, 1e-6, f"d{name} entrywise T={T}")


def check_grad_softmax_limits(grd):
    """(b1,b2) = (N,1) for any tiles and (1,N): exact attention, exact gradient."""
    import torch.nn.functional as F

    def sdpa(tq, tk, tv):
        return F.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None])[0, 0]

    for seed, (b1, b2, t, T) in enumerate([(12, 1, 1, 1), (12, 1, 5, 1), (1, 12, 1, 1), (12, 1, 3, 3),
                                            (1, 12, 1, 2)]):
        q, k, v, dy = _case(20 + seed, b1, b2, 8)
        got = grd.monarch_head_grad(q, k, v, dy, b1, b2, t, T)
        ref = _torch_grads(sdpa, q, k, v, dy)
        for name, a, b in zip("qkv", got, ref):
            _close(a, b, 1e-10, f"d{name} at (b1,b2,t,T)=({b1},{b2},{t},{T})")
    # one-row tiles with two or more iterations are exact attention too
    b1, b2 = 5, 4
    q, k, v, dy = _case(29, b1, b2, 6)
    ref = _torch_grads(sdpa, q, k, v, dy)
    for T in (2, 3):
        got = grd.monarch_head_grad(q, k, v, dy, b1, b2, b1, T)
        for name, a, b in zip("qkv", got, ref):
            _close(a, b, 1e-9, f"d{name} one-row tiles T={T}")


def check_grad_one_row_tiles(grd):
    """t = b1: y_n = sum_c1 softmax(s q Kbar)_c1 * sum_c2 softmax(s q k_c1)_c2 v_c1c2."""
    import torch

    b1, b2, d = 5, 4, 6

    def closed(tq, tk, tv):
        s = 1.0 / math.sqrt(d)
        kb = tk.reshape(b1, b2, d)
        vb = tv.reshape(b1, b2, d)
        lw = torch.softmax(s * tq @ kb.mean(dim=1).T, dim=-1)              # [N, c1]
        rw = torch.softmax(s * torch.einsum("nd,cpd->ncp", tq, kb), dim=-1)  # [N, c1, c2]
        return torch.einsum("nc,ncp,cpd->nd", lw, rw, vb)

    q, k, v, dy = _case(31, b1, b2, d)
    got = grd.monarch_head_grad(q, k, v, dy, b1, b2, b1)
    ref = _torch_grads(closed, q, k, v, dy)
    for name, a, b in zip("qkv", got, ref):
        _close(a, b, 1e-10, f"d{name} one-row tiles")


def check_grad_symmetries(grd):
    for seed, (b1, b2, t, d, T) in enumerate([(6, 5, 1, 8, 1), (6, 5, 3, 8, 1), (9, 4, 2, 4, 1), (6, 5, 3, 8, 2),
                                              (9, 4, 2, 4, 3)]):
        q, k, v, dy = _case(40 + seed, b1, b2, d)
        dq, dk, dv = grd.monarch_head_grad(q, k, v, dy, b1, b2, t, T)
        scale = np.max(np.abs(dk)) * k.shape[0]
        assert np.max(np.abs(dk.sum(axis=0))) <= 1e-11 * scale, "key shift: sum dk != 0"
        assert np.max(np.abs(dv.sum(axis=0) - dy.sum(axis=0))) <= 1e-11 * np.max(np.abs(dy)) * k.shape[0], \
            "value shift: sum dv != sum dy"
        a, b = float(np.sum(dq * q)), float(np.sum(dk * k))
        assert abs(a - b) <= 1e-10 * max(1.0, abs(a)), f"q/k scaling: {a} vs {b}"


def _chunk_case(seed, fk, fq, hw, d, scale=1.5):
    rng = np.random.default_rng(seed)
    N, Nq = fk * hw, fq * hw
    q = scale * rng.standard_normal((Nq, d))
    k = scale * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    dy = rng.standard_normal((Nq, d))
    return q, k, v, dy


def check_grad_chunk_directional_fd(grd):
    """Chunk of fq of fk frames (h*w tokens each), blocks (b1, b2) over all keys."""
    h = 1e-5
    for seed, (fk, fq, hw, b2, t, d, T) in enumerate([(4, 1, 12, 4, 1, 8, 1), (4, 2, 12, 4, 2, 8, 2),
                                                       (3, 1, 12, 6, 2, 4, 3), (5, 2, 6, 3, 4, 8, 1),
                                                       (4, 3, 8, 8, 3, 4, 2)]):
        q, k, v, dy = _chunk_case(70 + seed, fk, fq, hw, d)
        b1 = fk * hw // b2
        dq, dk, dv = grd.monarch_head_grad(q, k, v, dy, b1, b2, t, T)
        assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
        rng = np.random.default_rng(170 + seed)
        for which, g in (("q", dq), ("k", dk), ("v", dv)):
            args_p = {"q": q, "k": k, "v": v}
            u = rng.standard_normal(args_p[which].shape)
            args_m = dict(args_p)
            args_p[which] = args_p[which] + h * u
            args_m[which] = args_m[which] - h * u
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], dy, b1, b2, t, T)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], dy, b1, b2, t, T)) / (2 * h)
            an = float(np.sum(g * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                f"chunk d{which} (fk={fk},fq={fq},b2={b2},t={t},T={T}): fd {fd:.10f} vs analytic {an:.10f}"


def check_grad_chunk_softmax_limit(grd):
    """b2 = 1: every block holds one key, so the chunk's rows get exact
    attention over all keys, for any tiles and iterations."""
    import torch.nn.functional as F

    def sdpa(tq, tk, tv):
        return F.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None])[0, 0]

    for seed, (N, Nq, t, T) in enumerate([(20, 5, 1, 1), (20, 8, 3, 2), (15, 15, 2, 3)]):
        q, k, v, dy = _chunk_case(80 + seed, N, Nq, 1, 8)
        got = grd.monarch_head_grad(q, k, v, dy, N, 1, t, T)
        ref = _torch_grads(sdpa, q, k, v, dy)
        for name, a, b in zip("qkv", got, ref):
            _close(a, b, 1e-10, f"chunk d{name} at b2 = 1 (N={N}, Nq={Nq}, t={t}, T={T})")


def check_grad_chunk_is_last_tiles_of_full_layer(grd):
    """The last fq of fk frames with t tiles against all keys, and the square
    layer over all frames with t*fk/fq tiles (whose last t tiles cover the
    chunk with the same bounds) given dy = 0 outside the chunk: the same dk
    and dv, the chunk's dq on the chunk's rows and 0 on the others (tiles are
    independent query-row groups)."""
    fk, fq, h, w, d = 6, 2, 3, 4, 8
    b1, b2 = fk * h, w
    N, Nq = b1 * b2, fq * h * w
    rng = np.random.default_rng(90)
    q = 1.5 * rng.standard_normal((N, d))
    k = 1.5 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    dy = np.zeros((N, d))
    dy[N - Nq:] = rng.standard_normal((Nq, d))
    for t in (1, 2, 3):
        for T in (1, 2):
            fdq, fdk, fdv = grd.monarch_head_grad(q, k, v, dy, b1, b2, t * fk // fq, T)
            cdq, cdk, cdv = grd.monarch_head_grad(q[N - Nq:], k, v, dy[N - Nq:], b1, b2, t, T)
            scale = max(np.max(np.abs(fdk)), np.max(np.abs(fdq)), 1e-300)
            assert np.max(np.abs(fdq[:N - Nq])) <= 1e-13 * scale, (t, T, "dq outside the chunk")
            for name, a, b in (("dq", cdq, fdq[N - Nq:]), ("dk", cdk, fdk), ("dv", cdv, fdv)):
                _close(a, b, 1e-11, f"chunk {name} vs square layer (t={t}, T={T})")


ALL_CHECKS = [check_grad_directional_fd, check_grad_entrywise_fd, check_grad_softmax_limits,
              check_grad_one_row_tiles, check_grad_symmetries, check_grad_chunk_directional_fd,
              check_grad_chunk_softmax_limit, check_grad_chunk_is_last_tiles_of_full_layer]
