"""KDA forward oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package never
imports the product path.
"""
from .kda_oracle import build_oracle, oracle_fwd, oracle_threads  # noqa: F401
from .kda_oracle_bwd import forward_states, oracle_bwd  # noqa: F401,E402
