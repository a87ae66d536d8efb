"""CPU oracle for the Parallax attention operator (test infrastructure only).

Imported only by tests/, the smoke check and the benchmark's CPU-baseline leg.
It shares no code with the GPU library.
"""
from .parallax_oracle import (fwd, fwd_probe, bwd, bwd_probe, decode, decode_paged,  # noqa: F401
                              exact_lla_projector, visible_range, precision)
