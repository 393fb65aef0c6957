"""CPU oracle for paged-KV decode attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""

from .paged_attention import *  # noqa: F401,F403
from .paged_attention import __all__  # noqa: F401
