"""Chunked queries against cached keys on the GPU, against the CPU oracle
(needs an MI355X).

A chunk of fq frames attends to all f frames (cache plus itself); the oracle
reads the same bf16-rounded q (the last fq frames of the full draw), k, v.
Bars as for the square layer: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3 on
every output element of the compared heads, fp32 max-abs <= 1e-5.  The chunk
must also reproduce the matching rows of the full layer over all frames run
on the GPU with tiles that cover the chunk with the same bounds.
"""
import numpy as np
import pytest

import oracle
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, errors, say, to_device, to_host
from structured_attention_video_monarch_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_kv(wl, x, workspace=False):
    import structured_attention_video_monarch_amd as M
    q, k, v = (to_device(x, n, wl.dtype) for n in "qkv")
    out = torch.empty_like(q)
    ws = None
    if workspace:
        dt = M.MONARCH_BF16 if wl.dtype == "bf16" else M.MONARCH_F32
        nb = M.monarch_attn_kv_workspace_bytes(wl.B, wl.H, wl.fq, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2,
                                               wl.tiles, wl.iters, dt)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    M.monarch_attn_fwd_kv(q, k, v, out, wl.fq, wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters, workspace=ws)
    torch.cuda.synchronize()
    return to_host(out)


def compare_kv(wl, seed=0, heads=None, label="", workspace=False):
    say(f"[case] kv {label or wl.name} B={wl.B} H={wl.H} Nq={wl.Nq} N={wl.N} d={wl.d} "
        f"blocks=({wl.b1q}|{wl.b1},{wl.b2}) t={wl.tiles} T={wl.iters} {wl.dtype} seed={seed}")
    x = I.make_inputs(wl, seed)
    y = run_kv(wl, x, workspace)
    assert y.shape == (wl.B, wl.H, wl.Nq, wl.d) and np.all(np.isfinite(y))
    heads = range(wl.H) if heads is None else heads
    worst = (0.0, 0.0)
    for b in range(wl.B):
        for h in heads:
            ref = oracle.monarch_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], wl.b1, wl.b2, wl.tiles, wl.iters)
            mx, mean = errors(y[b, h], ref)
            worst = (max(worst[0], mx), max(worst[1], mean))
            if wl.dtype == "bf16":
                assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (b, h, mx, mean)
            else:
                assert mx <= F32_MAX_ABS, (b, h, mx)
    say(f"[ok] kv {label or wl.name}: max-abs {worst[0]:.3e} mean-abs {worst[1]:.3e}")
    return y


def test_kv_chunk480p():
    compare_kv(I.get_workload("chunk480p_kv"), heads=[0, 11])


@pytest.mark.parametrize("t,T", [(3, 1), (2, 2)])
def test_kv_chunk480p_tiles_iters(t, T):
    compare_kv(I.get_workload("chunk480p_kv").with_(H=2, tiles=t, iters=T), label=f"chunk480p_kv-t{t}-T{T}")


def test_kv_chunk720p():
    compare_kv(I.get_workload("chunk720p_kv"), heads=[0, 39], workspace=True)


KV_EDGE = [
    # name, B, H, d, f, fq, h, w, b1, b2, t, T, dtype
    ("one_frame_chunk", 1, 2, 64, 6, 1, 5, 12, 30, 12, 1, 1, "bf16"),
    ("b2_1_exact", 1, 2, 64, 5, 2, 3, 7, 105, 1, 2, 2, "bf16"),
    ("misaligned_blocks", 2, 2, 128, 6, 2, 4, 8, 48, 4, 3, 2, "bf16"),
    ("ragged_tiles_d16", 1, 3, 16, 7, 3, 5, 17, 35, 17, 4, 1, "bf16"),
    ("f32_small", 1, 2, 64, 6, 2, 3, 4, 18, 4, 2, 2, "f32"),
    ("f32_d128", 1, 1, 128, 4, 1, 9, 20, 36, 20, 3, 1, "f32"),
]


@pytest.mark.parametrize("case", KV_EDGE, ids=[c[0] for c in KV_EDGE])
def test_kv_edge_shapes(case):
    name, B, H, d, f, fq, h, w, b1, b2, t, T, dt = case
    compare_kv(I.Workload(name, B, H, d, f, h, w, b1, b2, t, T, dt, fq=fq), seed=4, label=name)


@pytest.mark.parametrize("T", [1, 2])
def test_kv_chunk_equals_rows_of_full_layer(T):
    """Chunk of the last 3 of 21 frames with 1 tile == the last of 7 tiles of
    the full layer over all 21 frames (both on the GPU)."""
    import structured_attention_video_monarch_amd as M
    wl = I.get_workload("chunk480p_kv").with_(H=2, iters=T)
    x = I.make_inputs(wl.with_(fq=0), 2)
    q_all, k, v = (to_device(x, n, "bf16") for n in "qkv")
    full = torch.empty_like(q_all)
    M.monarch_attn_fwd(q_all, k, v, full, wl.f, wl.h, wl.w, wl.b1, wl.b2, 7, T)
    q = q_all[:, :, wl.N - wl.Nq:].contiguous()
    out = torch.empty_like(q)
    M.monarch_attn_fwd_kv(q, k, v, out, wl.fq, wl.f, wl.h, wl.w, wl.b1, wl.b2, 1, T)
    torch.cuda.synchronize()
    d = (out.float() - full[:, :, wl.N - wl.Nq:].float()).abs().max().item()
    say(f"[ok] kv chunk vs full-layer rows T={T}: max-abs {d:.3e}")
    assert d <= 1e-6
