"""CPU oracle (float64 numpy) for the tiled MonarchAttention forward and the
gradient of its one-iteration form.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use it; the GPU library does not.
"""
from .monarch_oracle import *  # noqa: F401,F403
from .monarch_grad import *  # noqa: F401,F403
