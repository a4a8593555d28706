"""Plain CPU reference for the TurboQuant compressed KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
product path (the HIP library and its Python binding) never imports, links or
runs it, and this package imports nothing from the product path.
"""

from .tq_oracle import *  # noqa: F401,F403
