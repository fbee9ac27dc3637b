"""fp64 CPU oracle for CPR Gated DeltaNet -- test infrastructure only.

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py``.  The GPU product path never imports, calls or links anything here.
"""
from .gdn_backward_oracle import gdn_varlen_backward, recurrence_backward
from .gdn_oracle import (bf16_bits_to_f64, boundary_positions, gdn_varlen, num_boundary_rows,
                         recurrence, round_to_bf16)

__all__ = ["bf16_bits_to_f64", "boundary_positions", "gdn_varlen", "num_boundary_rows", "recurrence",
           "round_to_bf16", "recurrence_backward", "gdn_varlen_backward"]
