"""The forward captured in a HIP graph and replayed (needs an MI355X).

Callers that launch many small layers (a chunk of three frames is launch
bound: five kernels of 10-20 us each) can capture the workspace entry points,
which allocate nothing and record no memset, in a graph and replay it (the
early-stopping entry point included).  Each
case captures one call, then replays it three times with eager work of the
program and a synchronisation between the replays, and checks every replay
bit for bit against the eager result of the same call; the eager result is
checked against the oracle on one head with the usual bars.
"""
import numpy as np
import pytest

import oracle
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, errors, say, to_device, to_host
from structured_attention_video_monarch_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _layer(wl):
    """(workspace bytes, call(q, k, v, out, ws)) of the workload's entry point."""
    import structured_attention_video_monarch_amd as M
    if wl.kv:
        nb = M.monarch_attn_kv_workspace_bytes(wl.B, wl.H, wl.fq, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles,
                                               wl.iters)
        return nb, lambda q, k, v, out, ws: M.monarch_attn_fwd_kv(q, k, v, out, wl.fq, wl.f, wl.h, wl.w, wl.b1,
                                                                 wl.b2, wl.tiles, wl.iters, workspace=ws)
    nb = M.monarch_attn_workspace_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles, wl.iters)
    return nb, lambda q, k, v, out, ws: M.monarch_attn_fwd_ws(q, k, v, out, wl.f, wl.h, wl.w, wl.b1, wl.b2,
                                                             wl.tiles, wl.iters, ws)


CASES = [
    ("chunk480p", {}),
    ("clip480p", {"H": 2, "iters": 2}),
    ("chunk480p_kv", {"H": 2}),
    ("clip480p_frames", {"H": 1}),
]


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, over):
    wl = I.get_workload(name).with_(**over)
    say(f"[case] graph {name} H={wl.H} T={wl.iters} blocks=({wl.b1},{wl.b2})")
    x = I.make_inputs(wl, 4)
    q, k, v = (to_device(x, n, wl.dtype) for n in "qkv")
    nb, call = _layer(wl)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    eager = torch.empty_like(q)
    call(q, k, v, eager, ws)
    torch.cuda.synchronize()

    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one call off the capture, as torch asks before capturing
        call(q, k, v, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q, k, v, out, ws)
    torch.cuda.synchronize()

    other = torch.empty_like(q)
    for rep in range(3):
        out.fill_(float("nan"))
        call(k[:, :, :q.shape[2]].contiguous(), q if not wl.kv else k, v, other, ws)  # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
    y = to_host(eager)
    ref = oracle.monarch_head(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], wl.b1, wl.b2, wl.tiles, wl.iters)
    mx, mean = errors(y[0, 0], ref)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    say(f"[ok] graph {name}: 3 replays equal to the eager call; eager vs oracle max-abs {mx:.3e}")


def test_graph_replays_match_eager_early_stopping():
    """The early-stopping entry point: the iteration counts are set by a fill
    kernel and stopped heads are skipped on the device, with no memset and no
    synchronisation, so it captures too. Every replay's output and counts
    equal the eager call's; the eager call matches the oracle's early stop."""
    import structured_attention_video_monarch_amd as M
    wl = I.get_workload("clip480p").with_(H=2, iters=5)
    tol = 1e-3
    say(f"[case] graph early stopping clip480p H={wl.H} max_iters={wl.iters} tol={tol}")
    x = I.make_inputs(wl, 5)
    q, k, v = (to_device(x, n, wl.dtype) for n in "qkv")
    nb = M.monarch_attn_adaptive_workspace_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles,
                                                 wl.iters)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def call(q_, k_, v_, out_, used_):
        M.monarch_attn_fwd_adaptive(q_, k_, v_, out_, wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters, tol,
                                    iters_used=used_, workspace=ws)

    eager, used_e = torch.empty_like(q), torch.empty((wl.B, wl.H), dtype=torch.int32, device="cuda")
    call(q, k, v, eager, used_e)
    torch.cuda.synchronize()
    out, used = torch.empty_like(q), torch.empty_like(used_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(q, k, v, out, used)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q, k, v, out, used)
    torch.cuda.synchronize()
    other, used_o = torch.empty_like(q), torch.empty_like(used_e)
    for rep in range(3):
        out.fill_(float("nan"))
        used.fill_(-1)
        call(k, q, v, other, used_o)  # eager work in between, other inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}: output differs from the eager call"
        assert torch.equal(used, used_e), f"replay {rep}: iteration counts differ"
    counts = used_e.cpu().numpy()
    for h in range(wl.H):
        ref, used_ref, _ = oracle.monarch_head_adaptive(x["q"][0, h], x["k"][0, h], x["v"][0, h], wl.b1, wl.b2,
                                                        wl.tiles, wl.iters, tol)
        assert int(counts[0, h]) == used_ref, (h, int(counts[0, h]), used_ref)
        mx, mean = errors(to_host(eager)[0, h], ref)
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (h, mx, mean)
    say(f"[ok] graph early stopping: 3 replays equal to the eager call; iterations {counts.tolist()}")


@pytest.mark.parametrize("name,over", [("clip480p", {"H": 2, "iters": 2}), ("clip480p_frames", {"H": 1})],
                         ids=["clip480p_T2", "clip480p_frames"])
def test_graph_replays_training_forward(name, over):
    """The training forward writes only the caller's output and state, so it
    captures too. Every replay's output and state equal the eager call's bit
    for bit, and the backward run from a replayed state gives the eager
    gradients bit for bit (the backward is deterministic)."""
    import structured_attention_video_monarch_amd as M
    wl = I.get_workload(name).with_(**over)
    say(f"[case] graph training forward {name} H={wl.H} T={wl.iters} blocks=({wl.b1},{wl.b2})")
    x = I.make_inputs(wl, 6)
    q, k, v = (to_device(x, n, wl.dtype) for n in "qkv")
    dy = to_device(I.make_cotangent(wl, 6), "dy", wl.dtype)
    args = (wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters)
    nb = M.monarch_attn_train_state_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles, wl.iters,
                                          M.MONARCH_BF16)

    def grads(out_, state_):
        g = [torch.empty_like(q) for _ in range(3)]
        M.monarch_attn_bwd(q, k, v, out_, dy, *g, *args, state_)
        torch.cuda.synchronize()
        return g

    # states start filled with one byte value, so that alignment padding the
    # forward never writes compares equal and every written byte is compared
    eager, st_e = torch.empty_like(q), torch.full((nb,), 255, dtype=torch.uint8, device="cuda")
    M.monarch_attn_fwd_train(q, k, v, eager, *args, st_e)
    torch.cuda.synchronize()
    g_eager = grads(eager, st_e)
    out, st = torch.empty_like(q), torch.full_like(st_e, 255)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.monarch_attn_fwd_train(q, k, v, out, *args, st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.monarch_attn_fwd_train(q, k, v, out, *args, st)
    torch.cuda.synchronize()
    other, st_o = torch.empty_like(q), torch.empty_like(st_e)
    for rep in range(3):
        out.fill_(float("nan"))
        st.fill_(255)
        M.monarch_attn_fwd_train(k, q, v, other, *args, st_o)  # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}: output differs"
        assert torch.equal(st, st_e), f"replay {rep}: training state differs"
    for name_g, a, b in zip(("dq", "dk", "dv"), grads(out, st), g_eager):
        assert torch.equal(a, b), f"{name_g} from the replayed state differs"
    say(f"[ok] graph training forward {name}: 3 replays equal to the eager call (output and "
        f"{nb} state bytes); gradients from the replayed state equal")
