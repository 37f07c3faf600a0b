"""CPU oracle of the SVG-EAR routed sparse-attention path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the HIP library never calls it.
"""
from .svgear_oracle import *  # noqa: F401,F403
