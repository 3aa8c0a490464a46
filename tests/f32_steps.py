"""The oracle's own steps evaluated in float32 (test helper, CPU only).

For strongly peaked softmaxes the layer is ill-conditioned: a relative
rounding error of the order of float32's moves the next L-step's logits by
about s|q||k| times as much, so any float32 evaluation of the method lands
visibly away from the float64 oracle.  How far the oracle's own steps land
when run in float32 is then the scale the fp32 GPU path is held to on such
inputs.  The modules below are the oracle sources with every
float64 array made float32 (nothing else changes); they are built from the
source text, as the planted-mistake tests build theirs.
"""
from __future__ import annotations

import os
import re
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_FWD = os.path.join(ROOT, "oracle", "monarch_oracle.py")
_GRAD = os.path.join(ROOT, "oracle", "monarch_grad.py")
_cache = {}


def _float32_source(src: str) -> str:
    src = src.replace("dtype=np.float64", "dtype=np.float32")
    # new arrays without a dtype: float32
    src = re.sub(r"np\.(empty|zeros)\(\(([^()]*)\)\)", r"np.\1((\2), dtype=np.float32)", src)
    src = re.sub(r"np\.zeros\(([A-Za-z_][A-Za-z_0-9.]*\.shape\[[^\]]*\])\)", r"np.zeros(\1, dtype=np.float32)", src)
    return src


def float32_steps():
    """(forward module, gradient module) evaluating the oracle's steps in float32."""
    if "mods" not in _cache:
        fwd = types.ModuleType("oracle_float32")
        exec(compile(_float32_source(open(_FWD).read()), _FWD + ":float32", "exec"), fwd.__dict__)
        gsrc = _float32_source(open(_GRAD).read())
        anchor = "from .monarch_oracle import _blocks, l_step, r_step, tile_bounds, uniform_R"
        assert gsrc.count(anchor) == 1
        grad = types.ModuleType("oracle_grad_float32")
        for name in ("_blocks", "l_step", "r_step", "tile_bounds", "uniform_R"):
            grad.__dict__[name] = getattr(fwd, name)
        exec(compile(gsrc.replace(anchor, ""), _GRAD + ":float32", "exec"), grad.__dict__)
        _cache["mods"] = (fwd, grad)
    return _cache["mods"]
