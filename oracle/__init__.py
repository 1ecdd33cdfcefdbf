"""CPU oracle for the Sherry 1.25-bit ternary linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
HIP library and its Python binding never import it, and it imports nothing from
them.
"""

from .sherry_oracle import *  # noqa: F401,F403
from .compare_oracle import *  # noqa: F401,F403
