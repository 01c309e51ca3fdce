"""CPU oracle for the block-scaled FP8 linear projection (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and this package imports
nothing from the product path.

Every function is pinned by ``tests/test_oracle_pins.py`` to facts that do not
come from the oracle itself (values the pages print, closed forms, library
special cases, brute force).  See ``bsf8_oracle`` for the function list.
"""
from .bsf8_oracle import *  # noqa: F401,F403
from .bsf8_oracle import __all__  # noqa: F401
