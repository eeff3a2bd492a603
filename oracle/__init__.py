"""fp64 CPU oracle for the Ulysses H3 hot path -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the product
library ``ulysses_layout_amd`` and never imports it.
"""
from .oracle import *  # noqa: F401,F403
from .oracle import build  # noqa: F401
