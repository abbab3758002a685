"""Seeded synthetic inputs for paged decode attention (tests and bench)."""
from .generate import (CONFIGS, PAD_ENTRY, Workload, llama2_7b, llama3_8b, make,
                       prefix_shared, qwen2_05b, random_paged, relabel_blocks,
                       round_to_dtype, tiny, unshare_blocks)

__all__ = ["CONFIGS", "PAD_ENTRY", "Workload", "llama2_7b", "llama3_8b", "make",
           "prefix_shared", "qwen2_05b", "random_paged", "relabel_blocks",
           "round_to_dtype", "tiny", "unshare_blocks"]
