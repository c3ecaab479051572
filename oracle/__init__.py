"""CPU oracle of the GIFT encode/decode path (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product library.
It shares no code with ``fac_whitening_amd``.
"""
from . import fp8, gift  # noqa: F401
