"""CPU oracle for the MSA training hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does, and this
package imports nothing from the product package.  Plain numpy in float64.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, finite differences, invariants and the dense
special case), except the proxy-gradient definition itself, which the pages do
not give (see the reading R8 in ``msa_oracle``): its finite-difference and
invariant pins check the code against that reading, not the reading against
the pages.
"""
from .msa_oracle import *  # noqa: F401,F403
from .msa_oracle import Config, Doc, doc_grid  # noqa: F401
