"""The factors L and R themselves on the GPU against the oracle's (needs an
MI355X), through the test-only export monarch_attn_debug_factors_f32.

The output parity of the other GPU tests checks y = P^T L P R v; here the
factors of the last iteration are compared element by element (fp32,
max-abs <= 1e-5) on small shapes: the tiny case, several tiles and
iterations, a chunk-sized layer and key blocks longer than 128 (the online
R-step).  Every row of L (over c1) and of R (over c2) must also sum to 1.
"""
import numpy as np
import pytest

import oracle
from gpu_util import say
from structured_attention_video_monarch_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32_FACTOR_MAX_ABS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (name, B, H, d, f, h, w, b1, b2, tiles, iters)
CASES = [
    ("tiny", 1, 1, 16, 2, 4, 4, 8, 4, 1, 1),
    ("tiny_t2_T2", 1, 2, 16, 2, 4, 4, 8, 4, 2, 2),
    ("small_t3_T3", 1, 2, 32, 2, 6, 10, 12, 10, 3, 3),
    ("d128_t4", 2, 1, 128, 3, 8, 12, 24, 12, 4, 1),
    ("offgrid_T2", 1, 2, 64, 2, 5, 12, 20, 6, 2, 2),
    ("long_blocks_T2", 1, 1, 32, 3, 5, 40, 3, 200, 1, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_factors_match_oracle(case):
    import structured_attention_video_monarch_amd as M
    name, B, H, d, f, h, w, b1, b2, t, T = case
    wl = I.Workload(name, B, H, d, f, h, w, b1, b2, t, T, "f32")
    say(f"[case] factors {name} B={B} H={H} N={wl.N} d={d} blocks=({b1},{b2}) t={t} T={T}")
    x = I.make_inputs(wl, 0)
    q, k, v = (torch.from_numpy(x[n]).cuda() for n in "qkv")
    L, R = M.monarch_attn_debug_factors_f32(q, k, v, f, h, w, b1, b2, t, T)
    torch.cuda.synchronize()
    L, R = L.cpu().numpy().astype(np.float64), R.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(L)) and np.all(np.isfinite(R))
    assert np.abs(L.sum(axis=-1) - 1.0).max() <= 1e-5
    assert np.abs(R.sum(axis=-1) - 1.0).max() <= 1e-5
    worst = (0.0, 0.0)
    for b in range(B):
        for hh in range(H):
            _, (Lr, Rr, _) = oracle.monarch_head(x["q"][b, hh], x["k"][b, hh], x["v"][b, hh], b1, b2, t, T,
                                                 return_factors=True)
            el = np.abs(L[b, hh] - Lr).max()
            er = np.abs(R[b, hh] - Rr).max()
            worst = (max(worst[0], el), max(worst[1], er))
            assert el <= F32_FACTOR_MAX_ABS and er <= F32_FACTOR_MAX_ABS, (b, hh, el, er)
    say(f"[ok] factors {name}: L max-abs {worst[0]:.3e}, R max-abs {worst[1]:.3e}")
