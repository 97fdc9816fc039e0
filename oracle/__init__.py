"""Plain fp64 CPU oracle for the Hogwild! concurrent-attention decode step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``shared_kv_cache_amd``) never imports, calls or links anything here, and
nothing here imports the product path: the two share no code.
"""

from .hogwild_oracle import *  # noqa: F401,F403
