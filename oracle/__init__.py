"""CPU oracle of the decode layer: plain, slow, float64, written from the pages.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it; the HIP product path never does,
and shares no code with it.
"""
from . import formats, layer  # noqa: F401
