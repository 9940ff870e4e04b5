"""CPU float64 oracle of the verification sampler (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import this package; the product path never does.
"""
from .specverify_oracle import *  # noqa: F401,F403
from .commit_oracle import commit_reference  # noqa: F401
from .tree_oracle import *  # noqa: F401,F403
