"""Seeded random shapes on the GPU against the CPU oracle (needs an MI355X).

Every case draws its shape from one seeded generator (the list of cases is
fixed): batch and heads, head dimension d in {16, 32, 64, 128}, a small
video (f, h, w), blocks (b1, b2) with b2 any divisor of N up to 128 (so the
blocks need not follow the frame grid), tiles, iterations 1-3 and the dtype;
chunk cases also draw the chunk's frame count.  The forward, the chunk
against cached keys and the backward through every iteration (square and
chunk) are compared
element by element with the same bars as the hand-picked cases
(test_gpu_parity, test_gpu_kv, test_gpu_backward).
"""
import numpy as np
import pytest

from structured_attention_video_monarch_amd import inputs as I
from test_gpu_backward import compare_grad
from test_gpu_kv import compare_kv
from test_gpu_parity import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw(kind, seed):
    rng = np.random.default_rng([7001, {"fwd": 0, "kv": 1, "bwd": 2, "bwdkv": 3}[kind], seed])
    chunk = kind in ("kv", "bwdkv")
    d = int(rng.choice([16, 32, 64, 128]))
    f, h, w = (int(rng.integers(1, hi + 1)) for hi in (4, 8, 20))
    if chunk and f == 1:
        f = 2
    N = f * h * w
    fq = int(rng.integers(1, f)) if chunk else 0
    Nq = fq * h * w if fq else N
    divisors = [x for x in range(1, min(N, 128) + 1) if N % x == 0 and Nq % x == 0]
    b2 = int(rng.choice(divisors))
    b1 = N // b2
    b1q = Nq // b2
    t = int(rng.integers(1, min(b1q, 8) + 1))
    T = int(rng.integers(1, 4))
    dtype = str(rng.choice(["bf16", "f32"]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    return I.Workload(f"fuzz-{kind}{seed}", B, H, d, f, h, w, b1, b2, t, T, dtype, fq=fq)


@pytest.mark.parametrize("seed", range(300))
def test_fuzz_forward(seed):
    wl = draw("fwd", seed)
    compare(wl, seed=seed, label=f"{wl.name} f,h,w=({wl.f},{wl.h},{wl.w})")


@pytest.mark.parametrize("seed", range(32))
def test_fuzz_chunk_against_cached_keys(seed):
    wl = draw("kv", seed)
    compare_kv(wl, seed=seed, label=f"{wl.name} fq/f={wl.fq}/{wl.f} h,w=({wl.h},{wl.w})")


@pytest.mark.parametrize("seed", range(64))
def test_fuzz_backward(seed):
    wl = draw("bwd", seed)
    compare_grad(wl, seed=seed, label=f"{wl.name} f,h,w=({wl.f},{wl.h},{wl.w})", iters=wl.iters)


@pytest.mark.parametrize("seed", range(24))
def test_fuzz_backward_chunk(seed):
    wl = draw("bwdkv", seed)
    compare_grad(wl, seed=seed, label=f"{wl.name} fq/f={wl.fq}/{wl.f} h,w=({wl.h},{wl.w})", iters=wl.iters)
