"""Host-side address translation for the cache write.

The flat slot of logical position p of a sequence is
block_table[p // B] * B + p % B: position p sits at offset p % B of logical
block p // B, which the sequence's block table maps to a physical block
("KV 캐시 관리와 PagedAttention", llm-systems-engineering.pages.dev, section
on linking token order to storage; positions and blocks count from 0).
The scheduler side computes these slots for the tokens of a step and hands
them to reshape_and_cache as its slot mapping.
"""
from __future__ import annotations

import numpy as np


def slot_mapping(block_tables: np.ndarray, seq: np.ndarray, pos: np.ndarray, block_size: int) -> np.ndarray:
    """int64 slots of tokens (seq[t], pos[t]); block_tables is [S, M] int32."""
    bt = np.asarray(block_tables)
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    if np.any(pos < 0) or np.any(pos // block_size >= bt.shape[1]):
        raise ValueError("position outside the block table")
    physical = bt[seq, pos // block_size].astype(np.int64)
    return physical * block_size + pos % block_size
