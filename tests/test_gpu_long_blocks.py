"""Key blocks longer than 128 tokens on the GPU (needs an MI355X), forward
and backward.

Blocks of whole frames, (b1, b2) = (f, h*w), and any other factorisation
with b2 > 128 run the R-step with the online softmax over blocks of 64 keys
(the kernel for shorter blocks keeps a whole block row per wave).  Compared
with the CPU oracle element by element: bf16 max-abs <= 2e-2 and mean-abs
<= 2e-3 as for every workload, and in addition mean-abs <= 2e-2 of the
reference's mean magnitude (softmaxes over thousands of keys give small
outputs, where the absolute bars alone would say little); fp32 max-abs <=
1e-5.  One key block, (1, N), is exact softmax attention: its output and its
gradients are checked against scaled dot-product attention (and autograd
through it) in float64 on the CPU, not against the oracle; so is the output
on an input whose logits split into a frame term plus a position term.
The gradients (dq, dk, dv through every iteration, square layer and chunk)
are compared with the gradient oracle with the bars of test_gpu_backward.
"""
import numpy as np
import pytest

import oracle
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, errors, say, to_device, to_host
from structured_attention_video_monarch_amd import inputs as I
from test_gpu_adaptive import check_against_oracle, run_adaptive
from test_gpu_backward import compare_grad
from test_gpu_kv import run_kv
from test_gpu_parity import run_gpu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REL_MEAN = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check(wl, x, y, heads, label):
    assert np.all(np.isfinite(y))
    worst = (0.0, 0.0, 0.0)
    for b in range(wl.B):
        for h in heads:
            ref = oracle.monarch_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], wl.b1, wl.b2, wl.tiles, wl.iters)
            mx, mean = errors(y[b, h], ref)
            rel = mean / np.abs(ref).mean()
            worst = (max(worst[0], mx), max(worst[1], mean), max(worst[2], rel))
            if wl.dtype == "bf16":
                assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS and rel <= REL_MEAN, (b, h, mx, mean, rel)
            else:
                assert mx <= F32_MAX_ABS, (b, h, mx)
    say(f"[ok] {label}: max-abs {worst[0]:.3e} mean-abs {worst[1]:.3e} relative mean {worst[2]:.3e}")


def compare_long(wl, seed=0, heads=None, label=""):
    label = label or wl.name
    say(f"[case] long blocks {label} B={wl.B} H={wl.H} N={wl.N} d={wl.d} blocks=({wl.b1},{wl.b2}) "
        f"t={wl.tiles} T={wl.iters} {wl.dtype} seed={seed}")
    x = I.make_inputs(wl, seed)
    y = run_gpu(wl, x)
    check(wl, x, y, range(wl.H) if heads is None else heads, label)


# (name, B, H, d, f, h, w, b1, b2, tiles, iters, dtype)
LONG_EDGE = [
    ("frames_f32_d32", 1, 2, 32, 3, 5, 40, 3, 200, 1, 1, "f32"),
    ("frames_f32_d32_t3_T3", 1, 2, 32, 3, 5, 40, 3, 200, 3, 3, "f32"),
    ("b2_129_f32_d16", 1, 2, 16, 3, 1, 129, 3, 129, 3, 2, "f32"),
    ("b2_130_bf16_d64", 1, 3, 64, 2, 5, 26, 2, 130, 1, 2, "bf16"),
    ("frames_bf16_d128_t2", 1, 2, 128, 4, 9, 33, 4, 297, 2, 2, "bf16"),
    ("half_frames_bf16_d64", 2, 2, 64, 3, 20, 20, 6, 200, 3, 1, "bf16"),
    ("f32_d128_T2", 1, 1, 128, 2, 8, 40, 2, 320, 1, 2, "f32"),
    ("f32_d64_b2_1000", 1, 1, 64, 2, 20, 50, 2, 1000, 2, 2, "f32"),
]


@pytest.mark.parametrize("case", LONG_EDGE, ids=[c[0] for c in LONG_EDGE])
def test_long_block_edge_shapes(case):
    name, B, H, d, f, h, w, b1, b2, t, T, dt = case
    compare_long(I.Workload(name, B, H, d, f, h, w, b1, b2, t, T, dt))


@pytest.mark.parametrize("T", [1, 2])
def test_clip480p_frames(T):
    wl = I.get_workload("clip480p_frames").with_(iters=T)
    if T > 1:
        wl = wl.with_(H=2)
    compare_long(wl, heads=[0, wl.H - 1])


def test_latent720p_frames_head():
    # the whole workload in the benchmark's launch configuration, one head checked
    wl = I.get_workload("latent720p_frames")
    compare_long(wl, heads=[wl.H - 1])


def test_chunk_against_cached_keys_long_blocks():
    for wl, heads in ((I.get_workload("chunk480p_kv_frames"), [0, 11]),
                      (I.Workload("kv_frames_f32", 1, 2, 32, 3, 5, 40, 3, 200, 1, 2, "f32", fq=1), [0, 1])):
        say(f"[case] long blocks kv {wl.name} Nq={wl.Nq} N={wl.N} blocks=({wl.b1q}|{wl.b1},{wl.b2}) "
            f"T={wl.iters} {wl.dtype}")
        x = I.make_inputs(wl, 0)
        y = run_kv(wl, x)
        check(wl, x, y, heads, f"kv {wl.name}")


@pytest.mark.parametrize("dtype,T", [("f32", 1), ("f32", 2), ("bf16", 1)])
def test_one_key_block_is_exact_attention(dtype, T):
    """(b1, b2) = (1, N): every L is 1, Qh = q, and R is the softmax of s q k^T
    over all keys, so the layer is softmax attention at any iteration count."""
    wl = I.Workload("one_block", 1, 2, 64, 2, 6, 50, 1, 600, 1, T, dtype)
    say(f"[case] one key block of {wl.N} keys, {dtype}, T={T}")
    x = I.make_inputs(wl, 3)
    y = run_gpu(wl, x)
    for h in range(wl.H):
        q, k, v = (torch.from_numpy(x[n][0, h]).to(torch.float64)[None, None] for n in "qkv")
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, 0].numpy()
        mx, mean = errors(y[0, h], ref)
        if dtype == "bf16":
            assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (h, mx, mean)
        else:
            assert mx <= F32_MAX_ABS, (h, mx)
    say(f"[ok] one key block {dtype} T={T}: max-abs {mx:.3e}")


@pytest.mark.parametrize("tol", [1e-3, -1.0])
def test_adaptive_long_blocks(tol):
    wl = I.Workload("adaptive_frames", 1, 3, 64, 4, 9, 33, 4, 297, 2, 1, "bf16")
    say(f"[case] adaptive long blocks max_iters=5 tol={tol}")
    x = I.make_inputs(wl, 1)
    y, used = run_adaptive(wl, x, 5, tol)
    if tol < 0:
        assert np.all(used == 5), used
    worst = check_against_oracle(wl, x, y, used, 5, tol, heads=range(wl.H))
    say(f"[ok] adaptive long blocks tol={tol}: iterations {used.tolist()}, max-abs {worst[0]:.3e}")


def draw_long(seed):
    """A seeded shape with a key block longer than 128 tokens."""
    rng = np.random.default_rng([7101, seed])
    while True:
        d = int(rng.choice([16, 32, 64, 128]))
        f, h, w = int(rng.integers(1, 5)), int(rng.integers(1, 13)), int(rng.integers(20, 90))
        N = f * h * w
        divisors = [x for x in range(129, min(N, 2048) + 1) if N % x == 0]
        if divisors:
            break
    b2 = int(rng.choice(divisors))
    b1 = N // b2
    t = int(rng.integers(1, b1 + 1))
    T = int(rng.integers(1, 4))
    dtype = str(rng.choice(["bf16", "f32"]))
    return I.Workload(f"fuzz-long{seed}", 1, int(rng.integers(1, 3)), d, f, h, w, b1, b2, t, T, dtype)


@pytest.mark.parametrize("seed", range(128))
def test_fuzz_long_blocks(seed):
    wl = draw_long(seed)
    compare_long(wl, seed=seed, label=f"{wl.name} f,h,w=({wl.f},{wl.h},{wl.w})")


@pytest.mark.parametrize("seed", range(100, 160))
def test_fuzz_long_blocks_backward(seed):
    """dq, dk and dv through every iteration of seeded long-block shapes
    against the gradient oracle (the bars of the hand-picked cases)."""
    wl = draw_long(seed)
    compare_grad(wl, seed=seed, label=f"{wl.name} f,h,w=({wl.f},{wl.h},{wl.w}) b2={wl.b2}", iters=wl.iters)


# (name, B, H, d, f, h, w, b1, b2, tiles, iters, dtype, query frames (0: all))
LONG_BWD = [
    ("bwd_frames_f32_d32", 1, 2, 32, 3, 5, 40, 3, 200, 1, 1, "f32", 0),
    ("bwd_frames_f32_d32_t3_T2", 1, 2, 32, 3, 5, 40, 3, 200, 3, 2, "f32", 0),
    ("bwd_b2_129_f32_d16_T3", 1, 2, 16, 3, 1, 129, 3, 129, 3, 3, "f32", 0),
    ("bwd_b2_130_bf16_d64_T2", 1, 3, 64, 2, 5, 26, 2, 130, 1, 2, "bf16", 0),
    ("bwd_frames_bf16_d128_t2", 1, 2, 128, 4, 9, 33, 4, 297, 2, 1, "bf16", 0),
    ("bwd_frames_bf16_d128_t2_T2", 1, 2, 128, 4, 9, 33, 4, 297, 2, 2, "bf16", 0),
    ("bwd_f32_d128_b2_320_T2", 1, 1, 128, 2, 8, 40, 2, 320, 1, 2, "f32", 0),
    ("bwd_kv_frames_f32_T2", 1, 2, 32, 3, 5, 40, 3, 200, 1, 2, "f32", 1),
    ("bwd_kv_frames_bf16", 1, 2, 64, 4, 9, 33, 4, 297, 1, 1, "bf16", 2),
]


@pytest.mark.parametrize("case", LONG_BWD, ids=[c[0] for c in LONG_BWD])
def test_bwd_long_blocks(case):
    name, B, H, d, f, h, w, b1, b2, t, T, dt, fq = case
    compare_grad(I.Workload(name, B, H, d, f, h, w, b1, b2, t, T, dt, fq=fq), iters=T)


def test_bwd_clip480p_frames():
    wl = I.get_workload("clip480p_frames").with_(H=2)
    compare_grad(wl, heads=[1])


@pytest.mark.parametrize("dtype,t", [("f32", 1), ("f32", 3), ("bf16", 1)])
def test_frame_separable_input_is_exact_attention(dtype, t):
    """Logits that split into a frame part plus a position part: attention is
    a frame softmax times a position softmax, which blocks of whole frames
    reproduce exactly in one iteration at any tile count (checked against
    scaled dot-product attention in float64, not against the oracle)."""
    import structured_attention_video_monarch_amd as M
    f, h, w, d1, d2 = 6, 10, 20, 32, 32
    hw = h * w
    rng = np.random.default_rng(12)
    qf, kf = rng.standard_normal((f, d1)), rng.standard_normal((f, d1))
    qp, kp = rng.standard_normal((hw, d2)), rng.standard_normal((hw, d2))
    q = 1.3 * np.concatenate([np.repeat(qf, hw, axis=0), np.tile(qp, (f, 1))], axis=1)
    k = 1.3 * np.concatenate([np.repeat(kf, hw, axis=0), np.tile(kp, (f, 1))], axis=1)
    v = rng.standard_normal((f * hw, d1 + d2))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tq, tk, tv = (torch.from_numpy(a).to(tdt).cuda()[None, None].contiguous() for a in (q, k, v))
    say(f"[case] frame-separable input, blocks ({f},{hw}), t={t}, {dtype}")
    out = torch.empty_like(tq)
    (M.monarch_attn_fwd if dtype == "bf16" else M.monarch_attn_fwd_f32)(tq, tk, tv, out, f, h, w, f, hw, t, 1)
    torch.cuda.synchronize()
    # the reference reads the values the GPU read (bf16-rounded for bf16)
    rq, rk, rv = (x[0, 0].to(torch.float64).cpu()[None, None] for x in (tq, tk, tv))
    ref = torch.nn.functional.scaled_dot_product_attention(rq, rk, rv)[0, 0].numpy()
    mx, mean = errors(out[0, 0].float().cpu().numpy().astype(np.float64), ref)
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    else:
        assert mx <= F32_MAX_ABS, mx
    say(f"[ok] frame-separable input t={t} {dtype}: max-abs {mx:.3e}")


# key block length -> (frames, height, width, heads); 16384 is the largest
# key block the library takes
ONE_BLOCK = {100: (1, 10, 10, 2), 600: (2, 6, 50, 2), 16384: (1, 128, 128, 1)}


@pytest.mark.parametrize("dtype,b2,T", [("f32", 600, 1), ("f32", 600, 2), ("bf16", 600, 2), ("f32", 100, 2),
                                        ("bf16", 100, 1), ("f32", 16384, 1), ("bf16", 16384, 2)])
def test_one_key_block_gradients_are_attention_gradients(dtype, b2, T):
    """(b1, b2) = (1, N) is softmax attention as a function of q, k and v, not
    only in value (every L is identically 1 and Qh = q), so its gradients are
    those of dense attention: checked against autograd through scaled
    dot-product attention in float64 on the CPU, not against the gradient
    oracle, for the online R-step (600 keys, and 16384, the largest key block)
    and the register-resident one (100 keys), with the bars of
    test_gpu_backward; the training forward's output against the same
    attention with the forward bars."""
    from test_gpu_backward import BF16_REL_MAX, BF16_REL_MEAN, F32_REL_MAX, rel_errors, run_train
    f, h, w, H = ONE_BLOCK[b2]
    wl = I.Workload("one_block_grad", 1, H, 64, f, h, w, 1, b2, 1, T, dtype)
    say(f"[case] gradients of one key block of {wl.N} keys, {dtype}, T={T}")
    x = I.make_inputs(wl, 5)
    dyx = I.make_cotangent(wl, 5)
    yg, dq, dk, dv = run_train(wl, x, dyx)
    worst = {}
    for hh in range(wl.H):
        q, k, v = (torch.from_numpy(x[n][0, hh]).to(torch.float64).requires_grad_() for n in "qkv")
        y = torch.nn.functional.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None])[0, 0]
        mx, mean = errors(yg[0, hh], y.detach().numpy())
        if dtype == "bf16":
            assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, ("y", hh, mx, mean)
        else:
            assert mx <= F32_MAX_ABS, ("y", hh, mx)
        worst["y"] = (max(worst.get("y", (0.0, 0.0))[0], mx), 0.0)
        y.backward(torch.from_numpy(dyx["dy"][0, hh]).to(torch.float64))
        for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), (q.grad, k.grad, v.grad)):
            mx, mean = rel_errors(got[0, hh], ref.numpy())
            wv = worst.get(name, (0.0, 0.0))
            worst[name] = (max(wv[0], mx), max(wv[1], mean))
            if dtype == "bf16":
                assert mx <= BF16_REL_MAX and mean <= BF16_REL_MEAN, (name, hh, mx, mean)
            else:
                assert mx <= F32_REL_MAX, (name, hh, mx)
    say(f"[ok] one key block gradients {dtype} N={wl.N} T={T}: " + ", ".join(
        f"{n} {'max-abs' if n == 'y' else 'rel-max'} {wv[0]:.2e}" for n, wv in worst.items()))


@pytest.mark.parametrize("dtype,T", [("bf16", 1), ("bf16", 2), ("f32", 1)])
def test_late_spikes_beyond_the_weight_range(dtype, T):
    """As the late-spike case below, with spikes so strong that their weight
    would overflow fp32 against the reference the stream started from: key
    300 lifts rows by about 70 log2 units and key 590 by about 140 (logits of
    about 50 and 100 nats).  The bf16 inference forward keeps its reference
    until a 32-key half's row sum passes 2^64, which these halves do (the
    second one by an infinite weight), so it takes its rescaling branch
    mid-stream for those rows only; fp32 takes its own (the step maximum).
    Outputs against scaled dot-product attention in float64 on the CPU with
    the usual bars."""
    N, d = 600, 64
    heads = [I.make_late_spike_head(s, N, d, spikes=((300, 100.0), (590, 200.0)), dtype=dtype) for s in (0, 1)]
    wl = I.Workload("late_spikes_big", 1, len(heads), d, 2, 6, 50, 1, N, 1, T, dtype, pos_amp=0.0)
    say(f"[case] overflowing late spikes in one key block of {N} keys, {dtype}, T={T}")
    x = {n: np.stack([hd[i] for hd in heads])[None] for i, n in enumerate("qkv")}
    if dtype == "bf16":
        for i, n in enumerate("qkv"):
            x[n + "_bits"] = np.stack([hd[3][i] for hd in heads])[None]
    y = run_gpu(wl, x)
    assert np.isfinite(y).all()
    for h in range(wl.H):
        q, k, v = (torch.from_numpy(x[n][0, h]).to(torch.float64) for n in "qkv")
        ref = torch.nn.functional.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None])[0, 0]
        mx, mean = errors(y[0, h], ref.numpy())
        say(f"[ok] overflowing late spikes head {h}: max-abs {mx:.3e} mean-abs {mean:.3e}")
        if dtype == "bf16":
            assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (h, mx, mean)
        else:
            assert mx <= F32_MAX_ABS, (h, mx)


@pytest.mark.parametrize("dtype,T", [("f32", 1), ("f32", 2), ("bf16", 1), ("bf16", 2)])
def test_late_spikes_move_the_streaming_maximum(dtype, T):
    """One key block of 600 keys (exact softmax attention) whose best key for
    every query comes late: keys 300 and 590 of the stream lift many rows'
    maxima by more than 8 log2 units in the middle and in the last 64-key
    step, so the online R-step moves its reference maximum and rescales the
    accumulators mid-stream for those rows, and keeps it for the others of the
    same wave.  The output and its gradients against scaled dot-product
    attention (and autograd through it) in float64 on the CPU: fp32 with the
    usual bars for the outputs and every gradient (the gradients run through
    the log-sum-exps the rescaled forward keeps).  bf16: the outputs with the
    usual bars; its gradients are reported, not held to the bf16 gradient
    bars, because the input is as ill-conditioned for them as the peaked
    softmaxes of test_gpu_backward: where a row's softmax is one-hot, dz =
    R (dR - rho) cancels almost exactly (dR ~ rho), and the spike keys'
    gradients (norms 16 and 28) sum such terms, so the bf16 roundings of dU,
    U and R leave a few per cent there (measured: relative max 1.5-4.5e-2,
    dq relative mean 4.4e-2)."""
    from test_gpu_backward import F32_REL_MAX, rel_errors, run_train
    N, d = 600, 64
    heads = [I.make_late_spike_head(s, N, d, dtype=dtype) for s in (0, 1)]
    wl = I.Workload("late_spikes", 1, len(heads), d, 2, 6, 50, 1, N, 1, T, dtype, pos_amp=0.0)
    say(f"[case] late spikes in one key block of {N} keys, {dtype}, T={T}")
    x = {n: np.stack([hd[i] for hd in heads])[None] for i, n in enumerate("qkv")}
    if dtype == "bf16":
        for i, n in enumerate("qkv"):
            x[n + "_bits"] = np.stack([hd[3][i] for hd in heads])[None]
    dyx = I.make_cotangent(wl, 2)
    y = run_gpu(wl, x)
    yg, dq, dk, dv = run_train(wl, x, dyx)
    for h in range(wl.H):
        q, k, v = (torch.from_numpy(x[n][0, h]).to(torch.float64).requires_grad_() for n in "qkv")
        ref = torch.nn.functional.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None])[0, 0]
        for label, got in (("forward", y), ("training forward", yg)):
            mx, mean = errors(got[0, h], ref.detach().numpy())
            say(f"[ok] late spikes {label} head {h}: max-abs {mx:.3e} mean-abs {mean:.3e}")
            if dtype == "bf16":
                assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (label, h, mx, mean)
            else:
                assert mx <= F32_MAX_ABS, (label, h, mx)
        ref.backward(torch.from_numpy(dyx["dy"][0, h]).to(torch.float64))
        for name, got, gref in zip(("dq", "dk", "dv"), (dq, dk, dv), (q.grad, k.grad, v.grad)):
            mx, mean = rel_errors(got[0, h], gref.numpy())
            say(f"[ok] late spikes {name} head {h}: relative max {mx:.3e} mean {mean:.3e}")
            if dtype == "f32":
                assert mx <= F32_REL_MAX, (name, h, mx)
