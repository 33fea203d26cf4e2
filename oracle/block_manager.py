"""Block manager of the paged KV cache -- TEST INFRASTRUCTURE ONLY.

A plain Python model of the host-side bookkeeping the pages describe. It is
the reference the library's native block manager is compared with; like the
rest of oracle/ it shares no code with the library and is imported only by
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg.

What it follows:
- The pool and its free queue: the physical KV memory is cut into fixed-size
  blocks once, and a request that needs room for new tokens takes
  ceil(tokens / block_size) blocks from the queue of free blocks; when the
  pool cannot cover that, the request is refused ("vLLM teardown" on
  arcyou.ai, section on paging the KV cache like virtual memory).
- Sequences and block tables: each sequence maps its logical blocks, in
  order, to physical blocks; a new block is taken only when the last one is
  full (paper notes "PagedAttention: Efficient Memory Management for Large
  Language Model Serving", sections 3.2 KV Cache Manager and 3.3 Decoding
  with PagedAttention and vLLM).
- fork / append / free are the three operations every decoding algorithm is
  expressed in (same notes, section 4.2): fork copies a sequence's table and
  adds one reference to each of its blocks (section 3.4.1); append writes
  the next token, taking a new block when the last is full, or copying the
  last block first when it is shared (copy-on-write: a new block, the old
  one's count minus one, then the write goes to the new block: section
  3.4.1, and "KV 캐시 관리와 PagedAttention", section on splitting a shared
  block when it must be written); free drops one reference from each of the
  sequence's blocks and returns the blocks that reach zero to the pool (notes
  section 3.4.2; "KV 캐시 관리와 PagedAttention", section on returning blocks
  after a request ends).

Readings where the pages are silent:
- The free queue is first-in first-out: blocks are taken from its front and
  returned to its back, a sequence's blocks in table order. Its initial order
  is the caller's (ascending by default), which lets a test lay out the
  pages' figures, whose block ids are illustrative.
- A batched append (one token for each of several sequences, as in a decode
  step) handles the sequences in the order given, so of k sequences sharing
  a partly filled last block the first k-1 copy it and the last writes in
  place (the page's second response writes without a copy once the count
  has dropped to one). It either completes for every sequence or, when the
  pool is short, changes nothing.
- Positions, blocks and slots count from 0; slot = block * block_size + offset.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(RuntimeError):
    """The free pool cannot cover the request; nothing was changed."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0 or max_blocks_per_seq <= 0:
            raise ValueError("sizes must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must list every block exactly once")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free: deque = deque(order)
        self.refcount: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        self._next_id = 0

    # ------------------------------------------------------------ queries
    def num_free(self) -> int:
        return len(self.free)

    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lengths[seq]

    def live(self) -> List[int]:
        return sorted(self.tables)

    def slot(self, seq: int, position: int) -> int:
        """Where position `position` of seq is stored."""
        b = self.block_size
        return self.tables[seq][position // b] * b + position % b

    # ------------------------------------------------------------ operations
    def _take(self) -> int:
        blk = self.free.popleft()
        self.refcount[blk] = 1
        return blk

    def add_sequence(self, num_tokens: int) -> int:
        """A new sequence whose first num_tokens positions (its prompt) get
        blocks at once: ceil(num_tokens / block_size) of them."""
        if num_tokens < 0:
            raise ValueError("num_tokens must be >= 0")
        need = -(-num_tokens // self.block_size)
        if need > self.max_blocks_per_seq:
            raise ValueError("sequence longer than a block table row")
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        seq = self._next_id
        self._next_id += 1
        self.tables[seq] = [self._take() for _ in range(need)]
        self.lengths[seq] = num_tokens
        return seq

    def fork(self, parent: int) -> int:
        """A new sequence sharing every block of `parent`."""
        table = self.tables[parent]
        for blk in table:
            self.refcount[blk] += 1
        child = self._next_id
        self._next_id += 1
        self.tables[child] = list(table)
        self.lengths[child] = self.lengths[parent]
        return child

    def _needs_block(self, seq: int, counts: Dict[int, int]) -> bool:
        """Whether appending one token to seq takes a block from the pool,
        given the reference counts in `counts` (updated as if it happened)."""
        n, b = self.lengths[seq], self.block_size
        if n % b == 0:
            return True
        last = self.tables[seq][n // b]
        c = counts.get(last, self.refcount[last])
        if c > 1:
            counts[last] = c - 1
            return True
        return False

    def append_slots(self, seqs: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Room for one more token in each sequence, in order. Returns the
        slot of each new token and the (src, dst) block copies the writes
        need first (copy-on-write)."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence may appear once per batch")
        for s in seqs:
            if s not in self.tables:
                raise KeyError(f"no live sequence {s}")
            if self.lengths[s] // self.block_size >= self.max_blocks_per_seq:
                raise ValueError(f"sequence {s} would outgrow its block table row")
        counts: Dict[int, int] = {}
        need = sum(self._needs_block(s, counts) for s in seqs)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        slots, copies = [], []
        b = self.block_size
        for s in seqs:
            n = self.lengths[s]
            table = self.tables[s]
            if n % b == 0:
                table.append(self._take())
            else:
                last = table[n // b]
                if self.refcount[last] > 1:
                    new = self._take()
                    self.refcount[last] -= 1
                    table[n // b] = new
                    copies.append((last, new))
            slots.append(table[n // b] * b + n % b)
            self.lengths[s] = n + 1
        return slots, copies

    def free_sequence(self, seq: int) -> None:
        for blk in self.tables.pop(seq):
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free.append(blk)
        del self.lengths[seq]
