"""CPU oracle (float64 numpy) for the tiled MonarchAttention forward and its
gradient through one or several unrolled iterations (square layer, or a
chunk of query frames against cached keys).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use it; the GPU library does not.
"""
from .monarch_oracle import *  # noqa: F401,F403
from .monarch_grad import *  # noqa: F401,F403
