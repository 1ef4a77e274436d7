"""CPU fp64 oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU library
and imports nothing from it.
"""
from .attention import (  # noqa: F401
    attention_fwd,
    below_or_on_diag,
    count_visible_pairs,
    key_positions,
    lazy_blockwise_fwd,
    query_positions,
    ring_order,
    skip_map_bruteforce,
    skip_map_closed,
    visible,
)
from .backward import attention_bwd  # noqa: F401
from .decode import decode_attention  # noqa: F401
from .feedforward import blockwise_ffn, ffn  # noqa: F401
