"""Backward pass on the GPU against the CPU gradient oracle (needs an MI355X).

The upstream gradient dy is seeded (inputs.make_cotangent); the oracle reads
the same bf16-rounded q, k, v, dy.  Gradients have no natural scale, so the
bars are relative to the reference tensor of each head:
  fp32 I/O:  max |g - ref| <= 2e-5 * max |ref|
  bf16 I/O:  max |g - ref| <= 4e-2 * max |ref|  and  mean |g - ref| <= 1.5e-2 * mean |ref|
(the bf16 path rounds the weights L, R, dl and dz to bf16 as MFMA operands and
stores Qh, U, dU and G in bf16: a few relative errors of 2^-9 on every term).
Large workloads run whole on the GPU; the oracle checks a subset of heads.
"""
import numpy as np
import pytest

import oracle
from gpu_util import say, to_device, to_host
from structured_attention_video_monarch_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32_REL_MAX = 2e-5
F32_MAX_ABS_FWD = 1e-5   # the forward's fp32 bar (test_gpu_parity)
BF16_REL_MAX = 4e-2
BF16_REL_MEAN = 1.5e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_train(wl, x, dyx, host=True):
    """(y, dq, dk, dv) of the training forward and the backward: float64 host
    arrays, or the device tensors themselves when host is False."""
    import structured_attention_video_monarch_amd as M
    q, k, v = (to_device(x, n, wl.dtype) for n in "qkv")
    dy = to_device(dyx, "dy", wl.dtype)
    dt = M.MONARCH_BF16 if wl.dtype == "bf16" else M.MONARCH_F32
    out = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if wl.kv:
        # a chunk of fq frames against all f frames
        nb = M.monarch_attn_train_state_bytes_kv(wl.B, wl.H, wl.fq, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2,
                                                 wl.tiles, wl.iters, dt)
        state = torch.empty(nb, dtype=torch.uint8, device="cuda")
        args = (wl.fq, wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters)
        M.monarch_attn_fwd_train_kv(q, k, v, out, *args, state)
        M.monarch_attn_bwd_kv(q, k, v, out, dy, dq, dk, dv, *args, state)
    else:
        nb = M.monarch_attn_train_state_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles,
                                              wl.iters, dt)
        state = torch.empty(nb, dtype=torch.uint8, device="cuda")
        args = (wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters)
        M.monarch_attn_fwd_train(q, k, v, out, *args, state)
        M.monarch_attn_bwd(q, k, v, out, dy, dq, dk, dv, *args, state)
    torch.cuda.synchronize()
    if not host:
        return out, dq, dk, dv
    return [to_host(t) for t in (out, dq, dk, dv)]


def rel_errors(got, ref):
    d = np.abs(got - ref)
    return float(d.max() / max(np.abs(ref).max(), 1e-30)), float(d.mean() / max(np.abs(ref).mean(), 1e-30))


def compare_grad(wl, seed=0, heads=None, label="", iters=1, x=None):
    wl = wl.with_(iters=iters)
    say(f"[case] bwd {label or wl.name} B={wl.B} H={wl.H} Nq={wl.Nq} N={wl.N} d={wl.d} blocks=({wl.b1},{wl.b2}) "
        f"t={wl.tiles} T={wl.iters} {wl.dtype} seed={seed}")
    if x is None:
        x = I.make_inputs(wl, seed)
    dyx = I.make_cotangent(wl, seed)
    y, dq, dk, dv = run_train(wl, x, dyx)
    for t in (y, dq, dk, dv):
        assert np.all(np.isfinite(t))
    heads = range(wl.H) if heads is None else heads
    worst = {}
    for b in range(wl.B):
        for h in heads:
            refs = oracle.monarch_head_grad(x["q"][b, h], x["k"][b, h], x["v"][b, h], dyx["dy"][b, h],
                                            wl.b1, wl.b2, wl.tiles, wl.iters)
            for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
                mx, mean = rel_errors(got[b, h], ref)
                w = worst.get(name, (0.0, 0.0))
                worst[name] = (max(w[0], mx), max(w[1], mean))
                if wl.dtype == "bf16":
                    assert mx <= BF16_REL_MAX and mean <= BF16_REL_MEAN, (name, b, h, mx, mean)
                else:
                    assert mx <= F32_REL_MAX, (name, b, h, mx)
    say(f"[ok] bwd {label or wl.name} T={wl.iters}: " + ", ".join(
        f"{n} rel-max {w[0]:.2e} rel-mean {w[1]:.2e}" for n, w in worst.items()))
    return worst


@pytest.mark.parametrize("t", [1, 2, 4])
def test_bwd_tiny_f32(t):
    compare_grad(I.get_workload("tiny").with_(tiles=t), label=f"tiny-t{t}")


def test_bwd_chunk480p_f32():
    compare_grad(I.get_workload("chunk480p").with_(H=2, dtype="f32"), label="chunk480p-f32")


def test_bwd_chunk480p_bf16():
    compare_grad(I.get_workload("chunk480p"), heads=[0, 5, 11])


@pytest.mark.parametrize("t", [1, 4, 8])
def test_bwd_clip480p_spikes_bf16(t):
    compare_grad(I.get_workload(f"clip480p_spikes_t{t}_T1"), heads=[0, 11])


def test_bwd_latent720p_bf16():
    compare_grad(I.get_workload("latent720p"), heads=[0, 39])


# ragged and degenerate shapes (one iteration): partial tiles of rows and
# keys, odd block sizes, one-row tiles, non-aligned blocks, B > 1
EDGE = [
    # name, B, H, d, f, h, w, b1, b2, t, dtype
    ("b2_1_dense_rows", 1, 2, 64, 2, 5, 7, 70, 1, 1, "bf16"),
    ("b1_1_dense_cols", 1, 2, 64, 1, 1, 100, 1, 100, 1, "bf16"),
    ("odd_blocks", 2, 3, 32, 3, 7, 13, 21, 13, 2, "bf16"),
    ("one_row_tiles", 1, 2, 128, 2, 3, 10, 6, 10, 6, "bf16"),
    ("misaligned_blocks", 1, 2, 128, 4, 6, 8, 48, 4, 3, "bf16"),
    ("b2_128", 1, 1, 128, 2, 2, 128, 4, 128, 1, "bf16"),
    ("b2_17_d16", 1, 3, 16, 5, 7, 17, 35, 17, 4, "bf16"),
    ("ragged_f32", 2, 2, 64, 3, 11, 9, 33, 9, 5, "f32"),
    ("d32_f32", 1, 2, 32, 2, 9, 20, 18, 20, 2, "f32"),
    ("d128_f32", 1, 1, 128, 3, 5, 24, 15, 24, 3, "f32"),
    ("b1_big_ragged", 1, 1, 128, 7, 37, 3, 259, 3, 3, "bf16"),
    # last 32-row block of a tile column with 1, 16 or 17 rows (the dU pass's
    # 16-row form), and (tile, 16-row) tasks of kb_rside_a that do not divide
    # evenly over its four waves
    ("tail_1_row", 1, 2, 128, 3, 11, 12, 33, 12, 1, "bf16"),
    ("tail_16_rows_uneven_tasks", 1, 2, 64, 5, 48, 20, 240, 20, 5, "bf16"),
    ("tail_17_rows", 1, 2, 32, 7, 7, 16, 49, 16, 1, "bf16"),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_bwd_edge_shapes(case):
    name, B, H, d, f, h, w, b1, b2, t, dt = case
    compare_grad(I.Workload(name, B, H, d, f, h, w, b1, b2, t, 1, dt), seed=3, label=name)


@pytest.mark.parametrize("iters", [1, 2, 3])
def test_train_forward_equals_forward_and_bwd_is_deterministic(iters):
    """The training forward runs the forward's kernels on the same
    (pre-scaled) block means and keeps its state on the side: its output
    equals the inference forward's bit for bit.  The backward is
    deterministic: two calls give the same bits."""
    import structured_attention_video_monarch_amd as M
    wl = I.get_workload("clip480p_spikes_t4_T1").with_(H=2)
    x = I.make_inputs(wl, 1)
    dyx = I.make_cotangent(wl, 1)
    q, k, v = (to_device(x, n, "bf16") for n in "qkv")
    dy = to_device(dyx, "dy", "bf16")
    args = (wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, iters)
    ref = torch.empty_like(q)
    M.monarch_attn_fwd(q, k, v, ref, *args)
    nb = M.monarch_attn_train_state_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles, iters)
    state = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    M.monarch_attn_fwd_train(q, k, v, out, *args, state)
    g1 = [torch.empty_like(q) for _ in range(3)]
    g2 = [torch.empty_like(q) for _ in range(3)]
    M.monarch_attn_bwd(q, k, v, out, dy, *g1, *args, state)
    M.monarch_attn_bwd(q, k, v, out, dy, *g2, *args, state)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


# ---- several iterations: the reverse runs back through every R-step and
# L-step (keys and entropies of each R-step feed the next L-step)
@pytest.mark.parametrize("t,T", [(1, 2), (2, 2), (4, 2), (2, 3), (4, 3)])
def test_bwd_iters_tiny_f32(t, T):
    compare_grad(I.get_workload("tiny").with_(tiles=t), label=f"tiny-t{t}", iters=T)


@pytest.mark.parametrize("T", [2, 3])
def test_bwd_iters_chunk480p_f32(T):
    compare_grad(I.get_workload("chunk480p").with_(H=2, dtype="f32"), label="chunk480p-f32", iters=T)


@pytest.mark.parametrize("T", [2, 3])
def test_bwd_iters_chunk480p_bf16(T):
    compare_grad(I.get_workload("chunk480p"), heads=[0, 11], iters=T)


@pytest.mark.parametrize("t", [4, 8])
def test_bwd_iters_clip480p_spikes_bf16(t):
    compare_grad(I.get_workload(f"clip480p_spikes_t{t}_T1"), heads=[0, 11], iters=2)


def test_bwd_iters_latent720p_bf16():
    compare_grad(I.get_workload("latent720p"), heads=[0, 39], iters=2)


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_bwd_iters_edge_shapes(case):
    name, B, H, d, f, h, w, b1, b2, t, dt = case
    compare_grad(I.Workload(name, B, H, d, f, h, w, b1, b2, t, 1, dt), seed=5, label=name, iters=2)


@pytest.mark.parametrize("case", [c for c in EDGE if c[0] in ("odd_blocks", "b2_17_d16", "ragged_f32",
                                                               "one_row_tiles")], ids=lambda c: c[0])
def test_bwd_three_iters_edge_shapes(case):
    name, B, H, d, f, h, w, b1, b2, t, dt = case
    compare_grad(I.Workload(name, B, H, d, f, h, w, b1, b2, t, 1, dt), seed=6, label=name, iters=3)


# ---- a chunk of frames against cached keys (queries: the chunk's rows;
# keys and values: all frames)
@pytest.mark.parametrize("T", [1, 2])
def test_bwd_kv_chunk480p_f32(T):
    compare_grad(I.get_workload("chunk480p_kv").with_(H=2, dtype="f32"), label="chunk480p_kv-f32", iters=T)


@pytest.mark.parametrize("T", [1, 2])
def test_bwd_kv_chunk480p_bf16(T):
    compare_grad(I.get_workload("chunk480p_kv"), heads=[0, 11], iters=T)


def test_bwd_kv_chunk720p_bf16():
    compare_grad(I.get_workload("chunk720p_kv"), heads=[0, 39])


KV_EDGE = [
    # name, B, H, d, fq, f, h, w, b1, b2, t, dtype
    ("one_frame_of_four", 1, 2, 64, 1, 4, 3, 10, 12, 10, 1, "bf16"),
    ("tiles_in_chunk", 2, 2, 32, 2, 5, 4, 6, 20, 6, 3, "bf16"),
    ("blocks_off_grid", 1, 3, 16, 2, 6, 2, 9, 36, 3, 4, "f32"),
    ("b2_1", 1, 2, 64, 1, 3, 5, 7, 105, 1, 2, "bf16"),
    ("b2_128_f32", 1, 1, 128, 1, 2, 1, 128, 2, 128, 1, "f32"),
]


@pytest.mark.parametrize("case", KV_EDGE, ids=[c[0] for c in KV_EDGE])
@pytest.mark.parametrize("T", [1, 2])
def test_bwd_kv_edge_shapes(case, T):
    name, B, H, d, fq, f, h, w, b1, b2, t, dt = case
    compare_grad(I.Workload(name, B, H, d, f, h, w, b1, b2, t, 1, dt, fq=fq), seed=4, label=name, iters=T)


def test_bwd_kv_chunk_matches_square_layer_rows():
    """The chunk's gradient against the square layer's over all frames with
    tiles that cover the chunk with the same bounds and dy = 0 outside the
    chunk, both on the GPU (fp32): same dk, dv; dq on the chunk's rows, 0
    elsewhere."""
    import structured_attention_video_monarch_amd as M
    fq, f, h, w, d, t, T = 2, 6, 3, 8, 64, 2, 2
    b1, b2 = f * h, w
    full = I.Workload("square", 1, 2, d, f, h, w, b1, b2, t * f // fq, T, "f32")
    chunk = full.with_(fq=fq, tiles=t)
    x = I.make_inputs(full, 9)
    N, Nq = full.N, chunk.Nq
    dyx = I.make_cotangent(chunk, 9)
    dy_full = np.zeros((1, 2, N, d), dtype=np.float32)
    dy_full[:, :, N - Nq:] = dyx["dy"]
    _, fdq, fdk, fdv = run_train(full, x, {"dy": dy_full})
    xc = {"q": x["q"][:, :, N - Nq:], "k": x["k"], "v": x["v"]}
    _, cdq, cdk, cdv = run_train(chunk, xc, dyx)
    assert np.max(np.abs(fdq[:, :, :N - Nq])) == 0.0
    for name, a, b in (("dq", cdq, fdq[:, :, N - Nq:]), ("dk", cdk, fdk), ("dv", cdv, fdv)):
        err = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)
        assert err <= 2e-6, (name, err)


def _scaled_inputs(wl, seed, alpha):
    """The workload's inputs with q and k scaled by alpha (logits by alpha^2),
    rounded again to the I/O dtype."""
    x = I.make_inputs(wl, seed)
    for n in "qk":
        val = (x[n] * alpha).astype(np.float32)
        if wl.dtype == "bf16":
            x[n + "_bits"] = I.round_to_bf16_bits(val)
            x[n] = I.bf16_bits_to_f32(x[n + "_bits"])
        else:
            x[n] = val
    return x


@pytest.mark.parametrize("T", [1, 2])
def test_bwd_peaked_softmax_bf16(T):
    """q and k doubled (logits x4, both factors close to one-hot): the usual bars."""
    wl = I.get_workload("chunk480p").with_(H=2, dtype="bf16")
    compare_grad(wl, seed=7, label="chunk480p q,k x2 bf16", iters=T, x=_scaled_inputs(wl, 7, 2.0))


# fp32 on strongly peaked inputs: the layer is ill-conditioned there (a
# relative error e in any intermediate moves the next L-step's logits by about
# s|q||k| e), so the bar is set by what float32 arithmetic alone does to the
# method: PEAKED_FACTOR times the distance between the oracle's own steps run
# in float32 (f32_steps) and in float64, and never below the usual fp32 bar.
# The factor covers the kernels' other summation order (products summed along
# d in MFMA chains), hardware exp2/log2 and logits kept in log2 units.
PEAKED_FACTOR = 10.0


@pytest.mark.parametrize("T", [1, 2])
def test_peaked_softmax_f32(T):
    from f32_steps import float32_steps
    f32_fwd, f32_grad = float32_steps()
    wl = I.get_workload("chunk480p").with_(H=2, dtype="f32", iters=T)
    say(f"[case] peaked softmax fp32: chunk480p q,k x3 T={T}")
    x = _scaled_inputs(wl, 7, 3.0)
    dyx = I.make_cotangent(wl, 7)
    y, dq, dk, dv = run_train(wl, x, dyx)
    for h in range(wl.H):
        q, k, v, dy = x["q"][0, h], x["k"][0, h], x["v"][0, h], dyx["dy"][0, h]
        y64 = oracle.monarch_head(q, k, v, wl.b1, wl.b2, wl.tiles, T)
        y32 = f32_fwd.monarch_head(q, k, v, wl.b1, wl.b2, wl.tiles, T)
        bar = max(F32_MAX_ABS_FWD, PEAKED_FACTOR * float(np.abs(y32 - y64).max()))
        err = float(np.abs(y[0, h] - y64).max())
        say(f"  head {h} y: max-abs {err:.3e}, float32 steps {np.abs(y32 - y64).max():.3e}, bar {bar:.3e}")
        assert err <= bar, ("y", h, err, bar)
        r64 = oracle.monarch_head_grad(q, k, v, dy, wl.b1, wl.b2, wl.tiles, T)
        r32 = f32_grad.monarch_head_grad(q, k, v, dy, wl.b1, wl.b2, wl.tiles, T)
        for name, got, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), r32, r64):
            e32 = rel_errors(a, b)[0]
            mx = rel_errors(got[0, h], b)[0]
            bar = max(F32_REL_MAX, PEAKED_FACTOR * e32)
            say(f"  head {h} {name}: rel-max {mx:.3e}, float32 steps {e32:.3e}, bar {bar:.3e}")
            assert mx <= bar, (name, h, mx, bar)
