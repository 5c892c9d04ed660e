"""CPU oracle for the NVFP4 W4A4 linear: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links it, and the two share no code.
"""
from .nvfp4 import *  # noqa: F401,F403
from .nvfp4 import __all__  # noqa: F401
