"""Gradients at full size, every head, through identities of the method
(needs an MI355X).

The CPU gradient oracle takes minutes per head at these sizes, so the
training configurations that bench.py times are checked on all heads through
facts that hold at any size, for any blocks, tiles and iterations, and for a
chunk of query frames against all keys (the oracle obeys them too: the
symmetry pins of the gradient oracle):

* adding one vector to every key leaves each softmax unchanged (the R-step's
  over a key block, and the L-step's over block means or aggregated keys,
  which move by the same vector), so sum_n dk_n = 0;
* rows of M sum to 1, so adding one vector to every value adds it to every
  output row: sum_n dv_n = sum_m dy_m;
* y is linear in v: <dv, v> = <dy, y>;
* every logit is a product of a query side and a key side, so q -> a q,
  k -> k / a leaves y unchanged: <dq, q> = <dk, k>.

Each residual is measured against the sum of the magnitudes of its terms
(per head; per feature for the two sums over tokens).  The error of a sum is
at most the sum of its terms' errors, so the elementwise bars of
test_gpu_backward, relative errors of about 1.5e-2 for bf16 and 2e-5 for
fp32, bound these ratios too; the bars below are those.
"""
import numpy as np
import pytest

from gpu_util import say
from structured_attention_video_monarch_amd import inputs as I
from test_gpu_backward import run_train

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BAR = {"bf16": 1.5e-2, "f32": 2e-5}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def identity_ratios(q, k, v, y, dy, dq, dk, dv):
    """Worst residual / magnitude of each identity over heads (and features)."""
    f = [t.double() for t in (q, k, v, y, dy, dq, dk, dv)]
    q, k, v, y, dy, dq, dk, dv = f
    out = {}
    out["sum dk = 0"] = (dk.sum(dim=2).abs() / dk.abs().sum(dim=2).clamp_min(1e-300)).max().item()
    out["sum dv = sum dy"] = ((dv.sum(dim=2) - dy.sum(dim=2)).abs()
                              / (dv.abs().sum(dim=2) + dy.abs().sum(dim=2)).clamp_min(1e-300)).max().item()
    lin = ((dv * v).sum(dim=(2, 3)) - (dy * y).sum(dim=(2, 3))).abs()
    out["<dv,v> = <dy,y>"] = (lin / ((dv * v).abs().sum(dim=(2, 3)) + (dy * y).abs().sum(dim=(2, 3)))).max().item()
    sc = ((dq * q).sum(dim=(2, 3)) - (dk * k).sum(dim=(2, 3))).abs()
    out["<dq,q> = <dk,k>"] = (sc / ((dq * q).abs().sum(dim=(2, 3)) + (dk * k).abs().sum(dim=(2, 3)))).max().item()
    return out


CASES = [
    ("latent720p_frames", {}),
    ("latent720p_frames", {"dtype": "f32"}),
    ("latent720p", {}),
    ("latent720p", {"iters": 2}),
    ("chunk720p_kv", {}),
]


@pytest.mark.parametrize("name,over", CASES, ids=[f"{c[0]}-{'-'.join(f'{a}{b}' for a, b in c[1].items())}"
                                                   for c in CASES])
def test_gradient_identities_full_size(name, over):
    wl = I.get_workload(name).with_(**over)
    say(f"[case] gradient identities {name} B={wl.B} H={wl.H} Nq={wl.Nq} N={wl.N} d={wl.d} "
        f"blocks=({wl.b1},{wl.b2}) t={wl.tiles} T={wl.iters} {wl.dtype}")
    x = I.make_inputs(wl, 2)
    dyx = I.make_cotangent(wl, 2)
    y, dq, dk, dv = run_train(wl, x, dyx, host=False)
    for t in (y, dq, dk, dv):
        assert torch.isfinite(t).all()
    from gpu_util import to_device
    q, k, v = (to_device(x, n, wl.dtype) for n in "qkv")
    dy = to_device(dyx, "dy", wl.dtype)
    r = identity_ratios(q, k, v, y, dy, dq, dk, dv)
    say(f"[ratios] {name} {wl.dtype} T={wl.iters}: " + ", ".join(f"{n} {val:.2e}" for n, val in r.items()))
    for n, val in r.items():
        assert val <= BAR[wl.dtype], (n, val)
    say(f"[ok] gradient identities {name} {wl.dtype} T={wl.iters}")
