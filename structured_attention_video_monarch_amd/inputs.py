"""Seeded synthetic Q/K/V shaped like video self-attention workloads.

This module holds no part of the attention method.  It only draws random
numbers, adds a periodic positional signal, plants optional sparse matches and
rounds to bf16, so the same inputs feed both the CPU oracle and the GPU path.
It imports nothing else from this package and nothing from ``oracle/``.

Why the inputs look like this: the MonarchRT pages describe 3D video
attention as a dense, periodic, separable positional pattern plus a few sparse
long-range semantic matches (yunpan.plus MonarchRT article, section on
deconstructing 3D attention, Fig. 5; atlas.scime.ai summary, "Approach").  The
positional term below is separable over the (frame, row, column) axes, and the
planted spikes are strong query->key matches across frames and columns.

Recipe per (batch b, head h), with ``rng = np.random.default_rng([seed, b, h])``:

1. ``q, k, v = rng.standard_normal((N, d), float32)`` drawn in that order.
2. Positional term (added to q and k, not v): channel ``j`` follows axis
   ``j mod 3`` (0 frame, 1 row, 2 column); ``r = j // 3``; ``m = ceil(d/3)``;
   ``omega = 10000 ** (-2*(r//2)/m)``; value ``amp*sin(omega*coord)`` for even
   ``r`` and ``amp*cos(omega*coord)`` for odd ``r``.
3. Optional spikes: ``round(frac*N)`` distinct query rows (without
   replacement).  Row ``i`` gets one key ``j`` uniform over tokens in another
   frame and another column; ``q_i += (10*sqrt(d)/|k_j|^2) * k_j``, which raises
   that logit by 10 at scale ``1/sqrt(d)``.
4. bf16 workloads round every value to bf16 (round to nearest even).

Token order is ``n = (fi*h + hi)*w + wi`` (column fastest); arrays are
``[B, H, N, d]`` contiguous.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "positional_term",
    "round_to_bf16_bits", "bf16_bits_to_f32", "make_head", "make_inputs",
    "make_cotangent", "make_underflow_head", "make_late_spike_head",
]


@dataclass(frozen=True)
class Workload:
    """One attention-layer call: shapes, block sizes, tiles, iterations."""
    name: str
    B: int
    H: int
    d: int
    f: int
    h: int
    w: int
    b1: int
    b2: int
    tiles: int
    iters: int
    dtype: str                # "f32" or "bf16": the I/O and compute type
    spike_frac: float = 0.0   # fraction of query rows with a planted match
    pos_amp: float = 0.5
    fq: int = 0               # query frames: 0 = all f frames (the square layer);
                              # else the last fq frames attend to all f (cached keys)

    @property
    def N(self) -> int:
        """Key (and value) tokens: all f frames."""
        return self.f * self.h * self.w

    @property
    def Nq(self) -> int:
        """Query (and output) tokens."""
        return (self.fq or self.f) * self.h * self.w

    @property
    def b1q(self) -> int:
        """Query blocks of b2 tokens."""
        return self.Nq // self.b2

    @property
    def kv(self) -> bool:
        return bool(self.fq) and self.fq != self.f

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads of the method's stated settings: a tiny case the oracle
# finishes instantly, a Self-Forcing-like 3-frame chunk at 480p latent size,
# a 21-frame 480p latent clip, the same clip with planted spikes for the tile
# sweep, and a 720p-scale latent with four tiles per aligned block.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 16, 2, 4, 4, 8, 4, 1, 1, "f32"),
    "chunk480p": Workload("chunk480p", 1, 12, 128, 3, 30, 52, 90, 52, 1, 1, "bf16"),
    "clip480p": Workload("clip480p", 1, 12, 128, 21, 30, 52, 630, 52, 1, 1, "bf16"),
    "latent720p": Workload("latent720p", 1, 40, 128, 21, 45, 80, 945, 80, 4, 1, "bf16"),
    # a 3-frame chunk (Self-Forcing's unit of generation) attending to 18
    # cached frames plus itself, at the 480p and 720p latent sizes
    "chunk480p_kv": Workload("chunk480p_kv", 1, 12, 128, 21, 30, 52, 630, 52, 1, 1, "bf16", fq=3),
    "chunk720p_kv": Workload("chunk720p_kv", 1, 40, 128, 21, 45, 80, 945, 80, 1, 1, "bf16", fq=3),
    # blocks of whole frames, (b1, b2) = (f, h*w): L mixes frames at one
    # position, R mixes the positions of one frame (the spatio-temporal
    # factorisation of the VMonarch abstract), at the 480p and 720p sizes
    "clip480p_frames": Workload("clip480p_frames", 1, 12, 128, 21, 30, 52, 21, 1560, 1, 1, "bf16"),
    "latent720p_frames": Workload("latent720p_frames", 1, 40, 128, 21, 45, 80, 21, 3600, 1, 1, "bf16"),
    "chunk480p_kv_frames": Workload("chunk480p_kv_frames", 1, 12, 128, 21, 30, 52, 21, 1560, 1, 1, "bf16", fq=3),
}
for _t in (1, 2, 4, 8):
    for _T in (1, 2):
        _n = f"clip480p_spikes_t{_t}_T{_T}"
        WORKLOADS[_n] = Workload(_n, 1, 12, 128, 21, 30, 52, 630, 52, _t, _T,
                                 "bf16", spike_frac=0.02)


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")


def positional_term(f: int, h: int, w: int, d: int, amp: float = 0.5) -> np.ndarray:
    """[N, d] float64 sinusoidal (frame, row, column) signal (recipe step 2)."""
    fi, hi, wi = np.meshgrid(np.arange(f), np.arange(h), np.arange(w), indexing="ij")
    coords = np.stack([fi.ravel(), hi.ravel(), wi.ravel()], axis=1).astype(np.float64)
    m = -(-d // 3)
    out = np.empty((f * h * w, d), dtype=np.float64)
    for j in range(d):
        axis, r = j % 3, j // 3
        omega = 10000.0 ** (-2.0 * (r // 2) / m)
        x = omega * coords[:, axis]
        out[:, j] = amp * (np.sin(x) if r % 2 == 0 else np.cos(x))
    return out


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _plant_spikes(rng, q, k, f, h, w, frac):
    N, d = q.shape
    n_spk = int(round(frac * N))
    if n_spk == 0:
        return
    if f < 2 or w < 2:
        raise ValueError("spikes need at least two frames and two columns")
    rows = rng.choice(N, size=n_spk, replace=False)
    fi = rows // (h * w)
    wi = rows % w
    # uniform over tokens in another frame and another column: the candidate
    # set is a product of (other frames) x (all rows) x (other columns)
    fj = rng.integers(0, f - 1, size=n_spk)
    fj = fj + (fj >= fi)
    hj = rng.integers(0, h, size=n_spk)
    wj = rng.integers(0, w - 1, size=n_spk)
    wj = wj + (wj >= wi)
    cols = (fj * h + hj) * w + wj
    kj = k[cols].astype(np.float64)
    gain = 10.0 * math.sqrt(d) / np.sum(kj * kj, axis=1)
    q[rows] = (q[rows].astype(np.float64) + gain[:, None] * kj).astype(np.float32)


def make_head(wl: Workload, seed: int, b: int, h: int, pos: np.ndarray | None = None):
    """float32 (q, k, v), each [N, d], for one (batch, head), before rounding."""
    N, d = wl.N, wl.d
    rng = np.random.default_rng([seed, b, h])
    q = rng.standard_normal((N, d), dtype=np.float32)
    k = rng.standard_normal((N, d), dtype=np.float32)
    v = rng.standard_normal((N, d), dtype=np.float32)
    if wl.pos_amp != 0.0:
        if pos is None:
            pos = positional_term(wl.f, wl.h, wl.w, d, wl.pos_amp)
        q = (q.astype(np.float64) + pos).astype(np.float32)
        k = (k.astype(np.float64) + pos).astype(np.float32)
    if wl.spike_frac > 0.0:
        _plant_spikes(rng, q, k, wl.f, wl.h, wl.w, wl.spike_frac)
    return q, k, v


def _input_workers() -> int:
    """Threads for making inputs: the cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(wl: Workload, seed: int = 0, heads=None, want_f32: bool = True,
                want_bits: bool = True):
    """Seeded inputs for a workload.

    Returns a dict with, for q, k and v:
      ``<x>``      float32 values ``[B, len(heads), N, d]`` exactly as the GPU
                   sees them (bf16-rounded for bf16 workloads), if ``want_f32``;
      ``<x>_bits`` uint16 bf16 bit patterns, same shape (bf16 workloads, if
                   ``want_bits``).
    ``heads`` selects a subset of head indices (default: all); each head's
    values do not depend on which other heads are generated.  For a chunk
    against cached keys (``wl.fq``), q holds the last fq frames' queries of
    the same draw (``[B, heads, Nq, d]``); k and v hold all frames.
    """
    heads = list(range(wl.H)) if heads is None else list(heads)
    N, d = wl.N, wl.d
    shape = (wl.B, len(heads), N, d)
    qshape = (wl.B, len(heads), wl.Nq, d)
    bf16 = wl.dtype == "bf16"
    out = {}
    for name in "qkv":
        shp = qshape if name == "q" else shape
        if want_f32:
            out[name] = np.empty(shp, dtype=np.float32)
        if bf16 and want_bits:
            out[name + "_bits"] = np.empty(shp, dtype=np.uint16)
    pos = positional_term(wl.f, wl.h, wl.w, d, wl.pos_amp) if wl.pos_amp else None

    def one(item):
        b, j, hh = item
        tensors = list(make_head(wl, seed, b, hh, pos))
        tensors[0] = tensors[0][N - wl.Nq:]
        for name, x in zip("qkv", tensors):
            if bf16:
                bits = round_to_bf16_bits(x)
                if want_bits:
                    out[name + "_bits"][b, j] = bits
                if want_f32:
                    out[name][b, j] = bf16_bits_to_f32(bits)
            elif want_f32:
                out[name][b, j] = x

    # heads are drawn from generators of their own and written to disjoint
    # slices, so they can be made concurrently (numpy releases the GIL in
    # the draws and array arithmetic); the values do not depend on the order
    items = [(b, j, hh) for b in range(wl.B) for j, hh in enumerate(heads)]
    workers = min(len(items), _input_workers())
    if workers > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, items))
    else:
        for it in items:
            one(it)
    return out


def make_cotangent(wl: Workload, seed: int = 0, heads=None, want_f32: bool = True,
                   want_bits: bool = True):
    """Seeded upstream gradient dLoss/dout for the backward pass: standard
    normal per (batch, head), from its own stream (``[seed, b, h, 1]``), in
    the same dict format as :func:`make_inputs` under the key ``dy``."""
    heads = list(range(wl.H)) if heads is None else list(heads)
    shape = (wl.B, len(heads), wl.Nq, wl.d)
    bf16 = wl.dtype == "bf16"
    out = {}
    if want_f32:
        out["dy"] = np.empty(shape, dtype=np.float32)
    if bf16 and want_bits:
        out["dy_bits"] = np.empty(shape, dtype=np.uint16)
    def one(item):
        b, j, hh = item
        x = np.random.default_rng([seed, b, hh, 1]).standard_normal((wl.Nq, wl.d), dtype=np.float32)
        if bf16:
            bits = round_to_bf16_bits(x)
            if want_bits:
                out["dy_bits"][b, j] = bits
            if want_f32:
                out["dy"][b, j] = bf16_bits_to_f32(bits)
        elif want_f32:
            out["dy"][b, j] = x

    items = [(b, j, hh) for b in range(wl.B) for j, hh in enumerate(heads)]
    workers = min(len(items), _input_workers())
    if workers > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, items))
    else:
        for it in items:
            one(it)
    return out


def make_underflow_head(seed: int, b1: int, b2: int, d: int, cstar: int, dtype: str = "f32"):
    """A head whose block ``cstar`` of keys is pushed far away from every query.

    Standard normal q, k, v (``default_rng([seed, 7])``, drawn in that order),
    then, in channel 0 only: every query is set to 2; key 0 of block
    ``cstar`` to +64 and its other keys to -2400 (``b2 >= 2``).  At scale
    ``1/sqrt(d)`` the mean key of that block then sits about
    ``2*(64 - 2400*(b2-1))/(b2*sqrt(d))`` nats (-892 at b2 = 4, d = 16) below
    every other block for every query, beyond where exp underflows in fp64
    and fp32 alike, while its key 0 is the best single match of every query
    (+32 nats at d = 16).  All set values are exact in bf16, and the queries
    keep a norm close to that of the standard normal draws.  ``dtype ==
    "bf16"`` rounds the draws to bf16 as :func:`make_inputs` does.  Returns
    float32 ``(q, k, v)`` of shape ``[b1*b2, d]`` and, for bf16, their bit
    patterns as a 4th item.
    """
    if b2 < 2 or not 0 <= cstar < b1:
        raise ValueError("need b2 >= 2 and 0 <= cstar < b1")
    N = b1 * b2
    rng = np.random.default_rng([seed, 7])
    q = rng.standard_normal((N, d), dtype=np.float32)
    k = rng.standard_normal((N, d), dtype=np.float32)
    v = rng.standard_normal((N, d), dtype=np.float32)
    q[:, 0] = 2.0
    k[cstar * b2:(cstar + 1) * b2, 0] = -2400.0
    k[cstar * b2, 0] = 64.0
    if dtype == "bf16":
        bits = [round_to_bf16_bits(x) for x in (q, k, v)]
        q, k, v = (bf16_bits_to_f32(x) for x in bits)
        return q, k, v, bits
    return q, k, v


def make_late_spike_head(seed: int, N: int, d: int, spikes=((300, 16.0), (590, 28.0)), dtype: str = "f32"):
    """A head whose best key for every query sits late in the key order.

    Standard normal q, k, v (``default_rng([seed, 11])``, drawn in that
    order), then a unit vector ``u`` along channel 0: every query gets
    ``+4 u`` and each spike key ``j`` of ``spikes`` (pairs ``(j, b)``) is set
    to ``b u`` in channel 0 only.  At scale ``1/sqrt(d)`` spike ``j``'s logit
    is about ``b (4 + z) / sqrt(d)`` nats for a query with ``z ~ N(0, 1)`` in
    channel 0 (14 nats for b = 28, d = 64), well above the few nats of the
    other keys, so a streaming softmax over the keys in order meets a new row
    maximum several log2 units higher at each spike.  ``dtype == "bf16"``
    rounds to bf16 as :func:`make_inputs` does.  Returns float32 ``(q, k,
    v)`` of shape ``[N, d]`` and, for bf16, their bit patterns as a 4th item.
    """
    rng = np.random.default_rng([seed, 11])
    q = rng.standard_normal((N, d), dtype=np.float32)
    k = rng.standard_normal((N, d), dtype=np.float32)
    v = rng.standard_normal((N, d), dtype=np.float32)
    q[:, 0] += 4.0
    for j, b in spikes:
        if not 0 <= j < N:
            raise ValueError("spike key out of range")
        k[j, :] = 0.0
        k[j, 0] = b
    if dtype == "bf16":
        bits = [round_to_bf16_bits(x) for x in (q, k, v)]
        q, k, v = (bf16_bits_to_f32(x) for x in bits)
        return q, k, v, bits
    return q, k, v
