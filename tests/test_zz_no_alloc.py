"""The forward that allocates nothing (static scratch array) against the
workspace entry point it is a variant of, through the C ABI (needs an MI355X).

Two calls in a row, the second on a smaller input, each compared with
monarch_attn_fwd_ws on the same inputs: the kernels are the same, so the
outputs must agree bit for bit (and therefore within the bf16 bars of the
oracle comparison too).  A shape whose workspace exceeds the array is refused
with MONARCH_ENOMEM and launches nothing.
"""
import pytest

from gpu_util import say, to_device
from structured_attention_video_monarch_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(wl, seed):
    import structured_attention_video_monarch_amd as M
    say(f"[case] no-alloc {wl.name} H={wl.H} N={wl.N} blocks=({wl.b1},{wl.b2}) t={wl.tiles} T={wl.iters} {wl.dtype}")
    x = I.make_inputs(wl, seed)
    q, k, v = (to_device(x, n, wl.dtype) for n in "qkv")
    args = (wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters)
    o_ws = torch.full_like(q, float("nan"))
    dt = M.MONARCH_BF16 if wl.dtype == "bf16" else M.MONARCH_F32
    nb = M.monarch_attn_workspace_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles, wl.iters, dt)
    assert 0 < nb <= M.MONARCH_SCRATCH_BYTES
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    M.monarch_attn_fwd_ws(q, k, v, o_ws, *args, ws)
    o_sc = torch.full_like(q, float("nan"))
    M.monarch_attn_fwd_scratch(q, k, v, o_sc, *args)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o_sc.float()).all())
    assert torch.equal(o_sc, o_ws)
    say(f"[ok] no-alloc {wl.name}: equal to the workspace entry point")


def test_two_calls_second_smaller():
    # the 3-frame 480p chunk at two iterations, then a smaller ragged layer
    _both(I.get_workload("chunk480p").with_(iters=2, tiles=2), seed=0)
    _both(I.Workload("small", 1, 3, 64, 2, 5, 7, 10, 7, 3, 1, "bf16"), seed=1)


def test_f32_then_smaller_bf16():
    _both(I.get_workload("tiny").with_(H=5, tiles=2, iters=3), seed=2)
    _both(I.Workload("smaller", 1, 2, 32, 1, 3, 8, 3, 8, 1, 2, "bf16"), seed=3)


def test_too_large_is_refused_and_launches_nothing():
    import structured_attention_video_monarch_amd as M
    # a shape whose workspace exceeds the array: 40 heads at the 720p latent
    big = I.get_workload("latent720p")
    nb = M.monarch_attn_workspace_bytes(big.B, big.H, big.f, big.h, big.w, big.d, big.b1, big.b2, big.tiles,
                                        big.iters, M.MONARCH_BF16)
    assert nb > M.MONARCH_SCRATCH_BYTES
    q = torch.zeros((1, big.H, big.N, big.d), dtype=torch.bfloat16, device="cuda")
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    out = torch.full_like(q, 7.0)
    with pytest.raises(M.MonarchError) as e:
        M.monarch_attn_fwd_scratch(q, k, v, out, big.f, big.h, big.w, big.b1, big.b2, big.tiles, big.iters)
    assert e.value.status == M.MONARCH_ENOMEM
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all())
