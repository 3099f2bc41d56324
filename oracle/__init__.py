"""CPU oracle (test infrastructure only): see ``oracle.atom_oracle``.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
import this package.  The HIP library never does.
"""
from . import atom_oracle  # noqa: F401
