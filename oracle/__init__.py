"""CPU oracle for the wave index. TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The HIP library never links, loads or calls it, and it
shares no code, header, table or helper with the HIP path: both sides only consume the same seeded
inputs from ``kv_vector_index_amd.synth``.

Everything here is plain NumPy in float64 (``wave_index.py``), written from the pages' description
of RetroInfer's wave index, step by step in the pages' order.  Each function cites the passage it
follows.  Parity status of every function is listed in the module header of ``wave_index.py``.
"""
from .wave_index import *  # noqa: F401,F403
