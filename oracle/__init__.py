"""CPU oracle for the VSA attention path (test infrastructure, not product code).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP path never calls it and shares no
code with it.
"""
from .vsa_oracle import *  # noqa: F401,F403
from .vsa_oracle import __all__  # noqa: F401
