"""CPU float64 attention oracle: test infrastructure, never part of the product.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import this package.
"""
from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    backward_head,
    dq_rows,
    forward_head,
    probs_head,
    visible,
)
from .kvcache import gather_kv, kvcache_forward  # noqa: F401
