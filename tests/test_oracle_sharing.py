"""Pins of oracle.shared_prefix, the oracle's definition of the prompt prefix
a group of forked samples holds in common (paper notes section 3.4.1
Parallel sampling: the samples point at the prompt's physical blocks; "KV
캐시 관리와 PagedAttention", sections on sharing the common KV of several
responses and on splitting a shared block that must be written).

The pins come from outside the function: forks and appends driven through
the oracle's block manager (itself pinned to the pages' walk-throughs),
whose tables fix what is shared; and the definition's properties checked by
numpy indexing on random tables -- every member maps [0, P) to the same
slots, P lies within every context, and the next whole unit is not common.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.block_manager import BlockManager

pytestmark = pytest.mark.filterwarnings("ignore")


def forked(prompt: int, samples: int, tails, block_size: int = 16):
    """A prompt forked into `samples` sequences, then each sample given its
    own tail of tokens (a decode step at a time, all samples together)."""
    m = BlockManager(4096, block_size, 256)
    root = m.add_sequence(prompt)
    seqs = [root] + [m.fork(root) for _ in range(samples - 1)]
    for step in range(max(tails) if len(tails) else 0):
        m.append_slots([s for s, t in zip(seqs, tails) if t > step])
    tables = np.full((samples, 256), -1, np.int32)
    for i, s in enumerate(seqs):
        tables[i, :len(m.table(s))] = m.table(s)
    lens = np.array([m.length(s) for s in seqs], np.int32)
    return tables, lens


def test_whole_prompt_blocks_are_shared_after_divergent_tails():
    # A 512-token prompt fills 32 blocks; the samples' own tokens go to new
    # blocks, so all 32 stay common.
    tables, lens = forked(512, 6, [1, 5, 16, 17, 40, 3])
    assert oracle.shared_prefix(tables, lens, range(6), 16) == 512


def test_partial_last_prompt_block_is_copied_on_write():
    # 500 tokens: the 32nd block holds 4. The first write into it copies it
    # for every sample but the last, which then owns it alone; 31 blocks
    # stay common.
    tables, lens = forked(500, 6, [2, 2, 7, 1, 30, 9])
    assert len({int(t) for t in tables[:, 31]}) == 6
    assert oracle.shared_prefix(tables, lens, range(6), 16) == 496


def test_a_shared_partial_block_does_not_count():
    # Forked but not yet written: all 32 blocks are common, yet the last
    # holds only 4 tokens, so only the 31 full ones count.
    tables, lens = forked(500, 3, [])
    assert (tables[0, :32] == tables[1, :32]).all()
    assert oracle.shared_prefix(tables, lens, range(3), 16) == 496


def test_whole_tiles_at_small_blocks():
    # Block size 4: 70 prompt tokens fill 17 blocks (68 tokens); the run is
    # cut to whole 16-token tiles: 64.
    tables, lens = forked(70, 4, [3, 1, 2, 8], block_size=4)
    assert oracle.shared_prefix(tables, lens, range(4), 4) == 64
    # With a 4-token unit the 17 whole blocks count.
    assert oracle.shared_prefix(tables, lens, range(4), 4, tile=4) == 68


def test_single_member_and_unrelated_sequences():
    tables, lens = forked(100, 1, [5])
    assert oracle.shared_prefix(tables, lens, [0], 16) == 96  # 105 tokens: 6 full blocks
    m = BlockManager(64, 16, 8)
    a, b = m.add_sequence(40), m.add_sequence(40)
    tables = np.array([m.table(a) + [-1] * 5, m.table(b) + [-1] * 5], np.int32)
    assert oracle.shared_prefix(tables, [40, 40], [0, 1], 16) == 0


@pytest.mark.parametrize("seed", range(40))
def test_definition_properties_on_random_tables(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([4, 8, 16, 32, 64]))
    M = int(rng.integers(1, 12))
    k = int(rng.integers(1, 6))
    base = rng.permutation(200)[:M].astype(np.int32)
    tables = np.tile(base, (k, 1))
    for i in range(k):  # each member diverges from some entry on
        cut = int(rng.integers(0, M + 1))
        tables[i, cut:] = rng.integers(200, 400, M - cut)
    lens = rng.integers(0, M * B + 1, k).astype(np.int32)
    P = oracle.shared_prefix(tables, lens, range(k), B)
    unit = B * 16 // math.gcd(B, 16)
    assert P % unit == 0 and 0 <= P <= lens.min()
    pos = np.arange(P)
    slots = tables[:, pos // B] * B + pos % B  # every member's slots of [0, P)
    assert (slots == slots[0]).all()
    nxt = np.arange(P, P + unit)
    grows = P + unit <= lens.min() and P + unit <= M * B and \
        (tables[:, nxt // B] * B + nxt % B == (tables[0, nxt // B] * B + nxt % B)).all()
    assert not grows, "the common run would extend by another whole unit"
