"""fp64 CPU oracle for the DFlash-style draft step (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, calls or links it, and shares no code with
it.
"""
from .ref import *  # noqa: F401,F403
