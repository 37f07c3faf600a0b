"""MI355X-native (gfx950) routed sparse attention: the SVG-EAR hot path.

The compute lives in ``libsvgear.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/svgear.h``); ``svgear`` is its ctypes binding and
``synth`` draws the seeded synthetic workloads.
"""
from .svgear import (  # noqa: F401
    SvgearError, budget_keys, lib, routed_attention, svgear_attend, svgear_cluster,
    svgear_attend_unpermute, svgear_permute, svgear_probe, svgear_route, svgear_unpermute,
)
