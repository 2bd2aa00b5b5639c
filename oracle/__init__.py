"""CPU oracle (test infrastructure): the slow reference used to check the GPU path.

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. The library never does.
"""

from . import fp8_attention  # noqa: F401  (fp8_attention.quantize, .forward, ...)
from . import softmax_attention  # noqa: F401  (softmax_attention.forward, .backward, ...)
from .sigmoid_attention import (  # noqa: F401
    backward,
    backward_rows,
    backward_varlen,
    default_scalars,
    forward,
    forward_rows,
    forward_varlen,
    head_backward,
    head_forward,
    pack,
    per_sample_bias,
    scores,
    sigmoid,
    tile_plan,
    unpack,
)
