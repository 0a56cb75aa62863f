"""Plain CPU oracle for the Domino draft-head path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from .domino_oracle import *  # noqa: F401,F403
from .domino_oracle import __all__  # noqa: F401
