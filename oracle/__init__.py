"""Float64 CPU oracle for exact attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP path.
"""
from .attention import (backward, backward_head, decode, decode_head, forward, forward_head,
                        probabilities, tile_map)

__all__ = ["forward", "forward_head", "backward", "backward_head", "decode", "decode_head",
           "probabilities", "tile_map"]
