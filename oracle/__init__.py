"""CPU fp64 oracle for the KDA forward pass (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU leg of ``bench.py``
may import this package.  The GPU library never imports it and shares no code
with it.
"""
from .oracle import recurrence, chunked, num_chunks, load, qg, threads  # noqa: F401
