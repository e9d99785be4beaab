"""Float64 CPU oracle for exact attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP path.

``oracle.attention``: the plain definition (forward, backward, decode, tile map).
``oracle.fp8``: Q and K rotated by a random Hadamard matrix and quantised to
E4M3 per row, then the plain forward.
"""
from .attention import (backward, backward_head, decode, decode_head, forward, forward_head,
                        probabilities, tile_map)

__all__ = ["forward", "forward_head", "backward", "backward_head", "decode", "decode_head",
           "probabilities", "tile_map"]
