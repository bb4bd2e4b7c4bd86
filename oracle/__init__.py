"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library and its Python
binding never do, and the oracle never imports them.
"""
from . import sparse_decode  # noqa: F401
