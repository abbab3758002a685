"""CPU oracle (test infrastructure only): float64 paged decode attention and
the paged KV slot write, written from the pages' definitions.  Imported only by
the tests, the smoke check and the CPU-baseline leg of the bench."""
from . import block_manager_ref, paged_attention_ref

__all__ = ["block_manager_ref", "paged_attention_ref"]
