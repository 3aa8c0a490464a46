"""Helpers for the GPU parity tests: device upload and error measures."""
from __future__ import annotations

import sys

import numpy as np

BF16_MAX_ABS = 2e-2   # bf16 I/O: max |y_gpu - y_oracle|
BF16_MEAN_ABS = 2e-3  # bf16 I/O: mean |y_gpu - y_oracle|
F32_MAX_ABS = 1e-5    # fp32 path


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: dict, name: str, dtype: str):
    import torch
    if dtype == "bf16":
        bits = np.ascontiguousarray(x[name + "_bits"])
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x[name])).cuda()


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    return float(d.max()), float(d.mean())
