"""Plain CPU oracle for the paged-KV decode path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and has no CPU fallback.
"""

from .paged import *  # noqa: F401,F403
from . import paged  # noqa: F401
