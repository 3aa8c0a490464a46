"""The forward at full size, every head, through identities of the method
(needs an MI355X).

The oracle checks a few heads of each large workload; these checks cover
every head of the workloads bench.py times, in the launch form it times (the
workspace entry points), through facts that hold at any size:

* rows of M sum to 1, so values equal to one vector c per head give c on
  every output row.  The bf16 path rounds the weights of L and R to bf16 as
  MFMA operands (normalised by fp32 sums of the unrounded weights), stores
  R V in bf16 and rounds the output: four relative errors of at most 2^-9,
  so |y - c| <= 2^-7 |c| per feature;
* heads are independent: rolling the inputs over heads rolls the outputs,
  bit for bit;
* every logit is a product of a query side and a key side (L-step: queries
  with block means or aggregated keys; R-step: aggregated queries with
  keys), so q -> 2 q, k -> k / 2 leaves every logit, and y, unchanged.  A
  factor of two is exact in bf16 and commutes with every rounding of the
  path, so the outputs are equal bit for bit.
"""
import numpy as np
import pytest

from gpu_util import say, to_device
from structured_attention_video_monarch_amd import inputs as I
from test_gpu_graph import _layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# (workload, overrides); "tol" selects the early-stopping entry point with
# iters as the iteration cap (bench.py --iters 10 --tol 1e-3)
WORKLOADS = [("latent720p", {}), ("latent720p", {"iters": 2}), ("latent720p_frames", {}), ("chunk720p_kv", {}),
             ("latent720p", {"iters": 10, "tol": 1e-3})]
IDS = [f"{n}-T{o.get('iters', 1)}" + (f"-tol{o['tol']:g}" if "tol" in o else "") for n, o in WORKLOADS]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _adaptive_layer(wl, tol):
    """(workspace bytes, call) of the early-stopping entry point; the call
    also returns the iterations each head used."""
    import structured_attention_video_monarch_amd as M
    nb = M.monarch_attn_adaptive_workspace_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles,
                                                 wl.iters)
    return nb, lambda q, k, v, out, ws: M.monarch_attn_fwd_adaptive(q, k, v, out, wl.f, wl.h, wl.w, wl.b1, wl.b2,
                                                                    wl.tiles, wl.iters, tol, workspace=ws)[1]


def _setup(name, over, seed):
    over = dict(over)
    tol = over.pop("tol", None)
    wl = I.get_workload(name).with_(**over)
    say(f"[case] forward identities {name} B={wl.B} H={wl.H} Nq={wl.Nq} N={wl.N} d={wl.d} "
        f"blocks=({wl.b1},{wl.b2}) t={wl.tiles} T={wl.iters} tol={tol} {wl.dtype}")
    x = I.make_inputs(wl, seed)
    q, k, v = (to_device(x, n, wl.dtype) for n in "qkv")
    nb, call = _layer(wl) if tol is None else _adaptive_layer(wl, tol)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    used = []  # iterations per head of each run (early stopping only)

    def run(q_, k_, v_):
        out = torch.empty_like(q_)
        u = call(q_, k_, v_, out, ws)
        torch.cuda.synchronize()
        if tol is not None:
            used.append(u.clone())
        return out

    return wl, q, k, v, run, used


@pytest.mark.parametrize("name,over", WORKLOADS, ids=IDS)
def test_constant_values_pass_through(name, over):
    wl, q, k, v, run, _ = _setup(name, over, 3)
    c = v[:, :, :1, :]                      # one bf16 row per (batch, head)
    y = run(q, k, c.expand_as(v).contiguous()).double()
    cd = c.double()
    err = (y - cd).abs()
    ratio = (err / cd.abs().clamp_min(1e-30)).max().item()
    assert torch.isfinite(y).all()
    assert (err <= 2.0 ** -7 * cd.abs() + 1e-30).all(), ratio
    say(f"[ok] constant values {name} T={wl.iters}: max |y - c| / |c| = {ratio:.2e} over {wl.B * wl.H} heads")


@pytest.mark.parametrize("name,over", WORKLOADS, ids=IDS)
def test_heads_independent_and_bilinear_logits(name, over):
    wl, q, k, v, run, used = _setup(name, over, 4)
    y = run(q, k, v)
    assert torch.isfinite(y).all()
    shift = wl.H // 3 + 1
    yr = run(*(torch.roll(t, shift, dims=1).contiguous() for t in (q, k, v)))
    assert torch.equal(yr, torch.roll(y, shift, dims=1)), "rolling the heads changed some head's output"
    ys = run((q * 2).contiguous(), (k * 0.5).contiguous(), v)
    assert torch.equal(q * 2 / 2, q) and torch.equal(k * 0.5 * 2, k)  # the scaling was exact
    assert torch.equal(ys, y), f"q*2, k/2 changed y: max diff {(ys.double() - y.double()).abs().max().item():.3e}"
    if used:
        assert torch.equal(used[1], torch.roll(used[0], shift, dims=1)) and torch.equal(used[2], used[0])
        say(f"[ok] iterations per head: {sorted(set(used[0].flatten().tolist()))}")
    say(f"[ok] heads rolled by {shift}, and q*2, k/2: {name} T={wl.iters} outputs equal bit for bit")
