"""Pins of the oracle's block manager (oracle/block_manager.py).

Sources of truth: the integers of the pages' worked examples
(tests/golden/worked_examples.json: block growth, a prompt followed by decode
steps, the copy-on-write walk-through with its reference counts and blocks
in use, block counts) and a brute-force definition of what the bookkeeping
must achieve: with token ids standing in for K/V, a cache written at the
returned slots and copied per the returned pairs reads back, for every live
sequence, exactly that sequence's own token history.
"""
import json
import os

import numpy as np
import pytest

from oracle.block_manager import BlockManager, OutOfBlocks

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def in_use(m: BlockManager) -> int:
    return m.num_blocks - m.num_free()


def test_growth_example():
    """Request B (7 tokens, table [3, 0]) grows to 9 tokens next to request C
    (6 tokens, table [1, 4]) in a pool of 6 blocks of 4: position 7 fills the
    last slot of block 0, position 8 takes a new block (block 5 in the
    figure; the free queue is laid out so that 5 is next)."""
    g = GOLDEN["growth"]
    m = BlockManager(6, g["block_size"], 4, free_order=[3, 0, 1, 4, 5, 2])
    b = m.add_sequence(7)
    c = m.add_sequence(6)
    assert m.table(b) == [3, 0] and m.table(c) == [1, 4]
    for step in g["steps"]:
        slots, copies = m.append_slots([b])
        assert copies == []
        assert m.table(b) == step["table_after"]
        assert slots == [step["flat_slot"]]
        assert m.length(b) == step["position"] + 1
    assert in_use(m) == 5


def test_prompt_then_decode_example():
    g = GOLDEN["prompt_then_decode"]
    B = g["block_size"]
    m = BlockManager(8, B, 4, free_order=[7, 1, 3, 0, 2, 4, 5, 6])
    s = m.add_sequence(g["prompt_tokens"])
    assert len(m.table(s)) == g["prompt_blocks"] and m.table(s) == g["table_after_prompt"]
    filled = lambda: [min(B, m.length(s) - B * i) for i in range(len(m.table(s)))]
    assert filled() == g["filled_after_prompt"]
    for step in g["decode_steps"]:
        slots, copies = m.append_slots([s])
        assert copies == [] and slots == [step["flat_slot"]]
        assert m.table(s) == step["table_after"] and filled() == step["filled_after"]


@pytest.mark.parametrize("batched", [False, True])
def test_copy_on_write_example(batched):
    g = GOLDEN["copy_on_write"]
    B = g["block_size"]
    m = BlockManager(6, B, 4)
    r1 = m.add_sequence(g["prefix_tokens"])
    r2 = m.fork(r1)
    assert m.table(r1) == m.table(r2) == g["shared_table"]
    assert in_use(m) == g["blocks_when_shared"]
    assert m.refcount[1] == g["refcount_block_1"]["before"]
    if batched:
        slots, copies = m.append_slots([r1, r2])
    else:
        s1, c1 = m.append_slots([r1])
        s2, c2 = m.append_slots([r2])
        slots, copies = s1 + s2, c1 + c2
    assert copies == [tuple(g["response_1"]["copy"])]
    assert slots == [g["response_1"]["flat_slot"], g["response_2"]["flat_slot"]]
    assert m.table(r1) == g["response_1"]["table_after"]
    assert m.table(r2) == g["response_2"]["table_after"]
    assert m.refcount[1] == g["refcount_block_1"]["after_copy"]
    assert m.refcount[0] == g["refcount_block_0_after"]
    assert in_use(m) == g["physical_blocks_in_use_after"]
    # Ending both responses returns every block to the pool.
    m.free_sequence(r1)
    assert in_use(m) == 2 and m.refcount[0] == 1
    m.free_sequence(r2)
    assert in_use(m) == 0 and sum(m.refcount) == 0


def test_block_counts():
    for case in GOLDEN["block_counts"]["cases"]:
        m = BlockManager(100, case["block_size"], 100)
        s = m.add_sequence(case["tokens"])
        assert len(m.table(s)) == case["blocks"]


def test_samples_share_the_prompt_until_they_write():
    """Parallel sampling: every sample's table points at the prompt's
    blocks, whose reference count is the number of samples; a full shared
    block stays shared and each sample gets its own next block."""
    m = BlockManager(32, 4, 8)
    p = m.add_sequence(8)  # two full blocks
    kids = [m.fork(p) for _ in range(2)]
    assert all(m.refcount[b] == 3 for b in m.table(p))
    slots, copies = m.append_slots([p] + kids)
    assert copies == []
    assert all(m.refcount[b] == 3 for b in m.table(p)[:2])
    assert len({m.table(s)[2] for s in [p] + kids}) == 3
    assert len(set(slots)) == 3


def test_pool_shortage_changes_nothing():
    m = BlockManager(3, 4, 8)
    a = m.add_sequence(6)
    b = m.fork(a)
    c = m.fork(a)
    before = (m.num_free(), list(m.refcount), {s: m.table(s) for s in (a, b, c)})
    with pytest.raises(OutOfBlocks):
        m.append_slots([a, b, c])  # two copies needed, one block free
    assert (m.num_free(), list(m.refcount), {s: m.table(s) for s in (a, b, c)}) == before
    with pytest.raises(OutOfBlocks):
        m.add_sequence(5)
    slots, copies = m.append_slots([a])  # one copy fits
    assert len(copies) == 1 and m.num_free() == 0


def random_walk(m: BlockManager, rng, steps: int):
    """Drive m with random adds, forks, appends and frees; check after every
    operation that each live sequence reads back its own history from a
    token-id cache written through the slots and copies m returns."""
    B = m.block_size
    cache = np.full(m.num_blocks * B, -1, dtype=np.int64)
    history = {}
    next_token = [0]

    def new_tokens(n):
        t = list(range(next_token[0], next_token[0] + n))
        next_token[0] += n
        return t

    def check():
        for s, hist in history.items():
            slots = [m.slot(s, p) for p in range(m.length(s))]
            assert [int(cache[x]) for x in slots] == hist, f"sequence {s}"
        total = sum(len(m.table(s)) for s in history)
        assert sum(m.refcount) == total
        referenced = {b for s in history for b in m.table(s)}
        assert referenced.isdisjoint(set(m.free)) and len(referenced) + m.num_free() == m.num_blocks

    for _ in range(steps):
        op = rng.random()
        live = list(history)
        try:
            if op < 0.15 or not live:
                n = int(rng.integers(0, 3 * B))
                s = m.add_sequence(n)
                toks = new_tokens(n)
                for p, t in enumerate(toks):
                    cache[m.slot(s, p)] = t
                history[s] = toks
            elif op < 0.3:
                parent = live[int(rng.integers(len(live)))]
                child = m.fork(parent)
                history[child] = list(history[parent])
            elif op < 0.4 and len(live) > 1:
                s = live[int(rng.integers(len(live)))]
                m.free_sequence(s)
                del history[s]
            else:
                batch = list(rng.permutation(live)[: int(rng.integers(1, len(live) + 1))])
                batch = [int(s) for s in batch if m.length(int(s)) // B < m.max_blocks_per_seq]
                if not batch:
                    continue
                slots, copies = m.append_slots(batch)
                for src, dst in copies:  # copies first, then the writes
                    cache[dst * B:(dst + 1) * B] = cache[src * B:(src + 1) * B]
                for s, x in zip(batch, slots):
                    t = new_tokens(1)[0]
                    cache[x] = t
                    history[s].append(t)
        except OutOfBlocks:
            pass
        check()


@pytest.mark.parametrize("seed", range(6))
def test_random_walk_keeps_every_history(seed):
    rng = np.random.default_rng(seed)
    random_walk(BlockManager(40, 4, 12, free_order=rng.permutation(40)), rng, 400)


# ------------------------------------------------------------------ mutants
# Plausible mistakes planted in a copy of the oracle's block manager (on the
# CPU): each must fail at least one of the pins above.

BM_SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                           "block_manager.py")).read()
BM_MUTANTS = {
    "fork_without_reference": ("            self.refcount[blk] += 1\n", "            pass\n"),
    "copy_keeps_old_count": ("                    self.refcount[last] -= 1\n", "                    pass\n"),
    "copy_when_count_is_one": ("if self.refcount[last] > 1:", "if self.refcount[last] >= 1:"),
    "never_copy": ("if self.refcount[last] > 1:", "if False:"),
    "free_returns_shared_blocks": ("            if self.refcount[blk] == 0:\n                self.free.append(blk)",
                                   "            self.free.append(blk)"),
    "new_block_one_token_late": ("if n % b == 0:\n                table.append", "if n % b == 1:\n                table.append"),
    "prompt_blocks_floor": ("need = -(-num_tokens // self.block_size)", "need = num_tokens // self.block_size"),
    "lifo_free_queue": ("blk = self.free.popleft()", "blk = self.free.pop()"),
}


def load_mutant(name):
    a, b = BM_MUTANTS[name]
    assert a in BM_SRC, name
    ns = {}
    exec(compile(BM_SRC.replace(a, b, 1), f"<mutant {name}>", "exec"), ns)
    return ns["BlockManager"], ns["OutOfBlocks"]


@pytest.mark.parametrize("name", sorted(BM_MUTANTS))
def test_block_manager_mutant_is_caught(name, monkeypatch):
    import oracle.block_manager as bm
    Mut, MutOut = load_mutant(name)
    monkeypatch.setitem(globals(), "BlockManager", Mut)
    monkeypatch.setitem(globals(), "OutOfBlocks", MutOut)
    pins = [test_growth_example, test_prompt_then_decode_example, lambda: test_copy_on_write_example(False),
            lambda: test_copy_on_write_example(True), test_block_counts, test_samples_share_the_prompt_until_they_write,
            test_pool_shortage_changes_nothing] + [lambda s=s: test_random_walk_keeps_every_history(s)
                                                   for s in range(6)]
    caught = 0
    for pin in pins:
        try:
            pin()
        except (Exception, pytest.fail.Exception):  # noqa: BLE001 -- any failure counts as caught
            caught += 1
    assert caught > 0, f"mutant {name} passed every pin"
    assert bm.BlockManager is not Mut
