"""CPU oracle for the hybrid MoE FFN block -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The product path (the HIP
library and its Python binding) never imports, calls or falls back to it.

See ``oracle/moe_ref.py`` for the definitions and the pages they follow.
"""
from .moe_ref import *  # noqa: F401,F403
from .moe_ref import __all__  # noqa: F401
