"""CPU fp64 oracle for the tiled attention forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package: only the
tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import or run it. It shares no code with the HIP library.
"""
from .attention import (attention_ref, attention_ref_bwd, attention_ref_decode,
                        attention_ref_lse, attention_ref_rows, attention_ref_varlen,
                        attention_ref_varlen_mods, attention_ref_varlen_rows)

__all__ = ["attention_ref", "attention_ref_bwd", "attention_ref_decode", "attention_ref_lse",
           "attention_ref_rows", "attention_ref_varlen", "attention_ref_varlen_mods",
           "attention_ref_varlen_rows"]
