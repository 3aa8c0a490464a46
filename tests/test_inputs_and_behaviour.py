"""Seeded input generator, and behaviour the pages describe (CPU only).

Behaviour: block-aligned factors approximate video attention better than
factors over a shuffled token order (yunpan.plus MonarchRT article,
"Innovation 1: block alignment", Fig. 7 and Fig. 1 second row), and more tiles
give more accuracy (same article, "Innovation 2: tiled Monarch
parameterisation"; atlas.scime.ai summary, "Surprising findings").
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from structured_attention_video_monarch_amd import inputs as I


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    ours = I.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = I.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_positional_term_is_separable():
    f, h, w, d = 3, 4, 5, 24
    pos = I.positional_term(f, h, w, d, 0.5)
    assert pos.shape == (f * h * w, d) and np.max(np.abs(pos)) <= 0.5
    G = pos @ pos.T                                  # token-token products
    G = G.reshape(f * h, w, f * h, w)
    # G[a1,a2,c1,c2] = A[a1,c1] + Bw[a2,c2]: second differences vanish
    sep = G - G[:, :1, :, :1] - G[:1, :, :1, :] + G[:1, :1, :1, :1]
    assert np.max(np.abs(sep)) <= 1e-12


def test_inputs_deterministic_and_head_independent():
    wl = I.get_workload("tiny").with_(H=3)
    a = I.make_inputs(wl, seed=0)
    b = I.make_inputs(wl, seed=0, heads=[2])
    assert np.array_equal(a["q"][:, 2:3], b["q"])
    c = I.make_inputs(wl, seed=1)
    assert not np.array_equal(a["k"], c["k"])
    wl16 = I.get_workload("chunk480p").with_(H=1, f=2, h=3, w=4, b1=6, b2=4)
    x = I.make_inputs(wl16, seed=0)
    assert x["q_bits"].dtype == np.uint16
    assert np.array_equal(I.bf16_bits_to_f32(x["v_bits"]), x["v"])


def test_planted_spikes_raise_one_logit_by_ten():
    wl = I.get_workload("clip480p_spikes_t1_T1").with_(H=1, f=3, h=4, w=6, b1=12, b2=6, dtype="f32")
    base = I.get_workload("clip480p_spikes_t1_T1").with_(H=1, f=3, h=4, w=6, b1=12, b2=6,
                                                          dtype="f32", spike_frac=0.0)
    qs, ks, _ = I.make_head(wl, 0, 0, 0)
    q0, k0, _ = I.make_head(base, 0, 0, 0)
    assert np.array_equal(ks, k0)
    changed = np.nonzero(np.any(qs != q0, axis=1))[0]
    assert len(changed) == round(0.02 * wl.N)
    d = wl.d
    for i in changed:
        gain = (qs[i].astype(np.float64) - q0[i]) @ ks.T.astype(np.float64) / math.sqrt(d)
        j = int(np.argmax(gain))
        assert abs(gain[j] - 10.0) < 1e-3
        fi, wi = i // (wl.h * wl.w), i % wl.w
        assert j // (wl.h * wl.w) != fi and j % wl.w != wi


def _kl_to_dense(q, k, v, b1, b2, t, T):
    d = q.shape[1]
    _, (L, R, _) = oracle.monarch_head(q, k, v, b1, b2, t, T, return_factors=True)
    M = oracle.dense_monarch_matrix(L, R, oracle.tile_bounds(b1, t))
    S = (q.astype(np.float64) @ k.T.astype(np.float64)) / math.sqrt(d)
    A = oracle.softmax(S, axis=-1)
    return float(oracle.row_kl(M, A).mean())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_aligned_blocks_beat_shuffled(seed):
    wl = I.get_workload("chunk480p").with_(H=1, f=3, h=10, w=12, b1=30, b2=12, dtype="f32")
    q, k, v = I.make_head(wl, seed, 0, 0)
    perm = np.random.default_rng(100 + seed).permutation(wl.N)
    kl_al = _kl_to_dense(q, k, v, wl.b1, wl.b2, 1, 1)
    kl_sh = _kl_to_dense(q[perm], k[perm], v[perm], wl.b1, wl.b2, 1, 1)
    assert kl_al < kl_sh, (kl_al, kl_sh)


def test_aligned_blocks_much_better_when_structure_dominates():
    wl = I.get_workload("chunk480p").with_(H=1, f=3, h=10, w=12, b1=30, b2=12, dtype="f32",
                                           pos_amp=1.0)
    q, k, v = I.make_head(wl, 0, 0, 0)
    q = (q - I.positional_term(3, 10, 12, 128, 1.0)) * 0.5 + I.positional_term(3, 10, 12, 128, 1.0)
    k = (k - I.positional_term(3, 10, 12, 128, 1.0)) * 0.5 + I.positional_term(3, 10, 12, 128, 1.0)
    perm = np.random.default_rng(7).permutation(wl.N)
    kl_al = _kl_to_dense(q, k, v, wl.b1, wl.b2, 1, 1)
    kl_sh = _kl_to_dense(q[perm], k[perm], v[perm], wl.b1, wl.b2, 1, 1)
    assert kl_sh >= 1.5 * kl_al, (kl_al, kl_sh)


def test_more_tiles_more_accuracy():
    wl = I.get_workload("clip480p_spikes_t1_T1").with_(H=1, f=3, h=16, w=20, b1=48, b2=20,
                                                       dtype="f32")
    q, k, v = I.make_head(wl, 0, 0, 0)
    for T in (1, 2):
        kls = [_kl_to_dense(q, k, v, wl.b1, wl.b2, t, T) for t in (1, 2, 4, 8)]
        assert all(b <= a + 1e-12 for a, b in zip(kls, kls[1:])), (T, kls)


def test_chunk_queries_are_the_tail_of_the_full_draw():
    from structured_attention_video_monarch_amd import inputs as I
    wl = I.Workload("kvsmall", 1, 2, 16, 6, 3, 4, 18, 4, 1, 1, "bf16", fq=2)
    x = I.make_inputs(wl, 5)
    full = I.make_inputs(wl.with_(fq=0), 5)
    assert x["q"].shape == (1, 2, 2 * 3 * 4, 16) and x["k"].shape == (1, 2, 6 * 3 * 4, 16)
    assert np.array_equal(x["q_bits"], full["q_bits"][:, :, -24:])
    assert np.array_equal(x["k_bits"], full["k_bits"]) and np.array_equal(x["v_bits"], full["v_bits"])


def test_float32_steps_helper_is_the_oracle_in_float32():
    """The float32 evaluation used as the scale for ill-conditioned fp32 cases
    computes the oracle's method: float32 results, within float32 rounding of
    the float64 oracle on ordinary inputs."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from f32_steps import float32_steps
    import oracle
    f32_fwd, f32_grad = float32_steps()
    rng = np.random.default_rng(3)
    b1, b2, t, d = 6, 4, 2, 8
    q, k, v, dy = (rng.standard_normal((b1 * b2, d)) for _ in range(4))
    for T in (1, 2):
        y32 = f32_fwd.monarch_head(q, k, v, b1, b2, t, T)
        y64 = oracle.monarch_head(q, k, v, b1, b2, t, T)
        assert y32.dtype == np.float32 and np.abs(y32 - y64).max() <= 1e-5
        for a, b in zip(f32_grad.monarch_head_grad(q, k, v, dy, b1, b2, t, T),
                        oracle.monarch_head_grad(q, k, v, dy, b1, b2, t, T)):
            assert a.dtype == np.float32 and np.abs(a - b).max() <= 1e-5 * max(1.0, np.abs(b).max())
