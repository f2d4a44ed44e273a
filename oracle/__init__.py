"""CPU oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg use it.
It shares no code with the HIP library; the two meet only in the seeded inputs of
``workloads``.

See ``oracle/attention.py`` for the definitions, the sources they follow and the
readings taken where the sources are silent.
"""
from .attention import (  # noqa: F401
    to_f64,
    head_forward,
    head_backward,
    forward,
    backward,
    backward_stats,
    forward_rows,
    backward_query_rows,
    backward_key_rows,
    head_decode,
    decode,
)
from .fp8 import e4m3_decode, forward_fp8  # noqa: F401
