"""Seeded synthetic inputs for paged decode attention and its companion calls.

This module is shared by the GPU path (tests, bench) and by the CPU oracle's
tests. It holds none of the method's arithmetic: it draws sequence lengths,
physical block placements and N(0, 1) tensors, casts them to the storage
dtype, and lays out block tables as lists of physical block ids. Translating a
token position into a cache slot, attention, cache writes and block copies are
left to the two sides (the HIP library and the oracle), each in its own code.

Shapes follow the OPT-13B layer used throughout the pages: 40 heads of 128,
block size 16 (PagedAttention paper review, mz-moonzoo.tistory.com/116,
section 3 on KV cache size; paper notes on unpurerationalist.github.io,
section 2 "Memory Challenges in LLM Serving").

Draw order for every workload: lengths, then the block permutation, then q,
then K, then V, then any new-token K and V. Everything is drawn in float32
and cast round-to-nearest-even to the storage dtype. bf16 tensors are held as
their uint16 bit patterns, because numpy has no bf16 type.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional, Sequence, Union

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# Storage numpy type per dtype name (bf16 as raw bits).
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
# Quiet-NaN encodings used to poison memory the kernels must never read.
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits.

    Valid for finite inputs, which is all the generators produce.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 data to the storage array of `dtype`."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_float32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a storage array back to float32 (exact for all three dtypes)."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x.astype(np.float32)


def poison(arr: np.ndarray, dtype: str, index) -> None:
    """Write NaN into `arr[index]` (storage array of `dtype`)."""
    if dtype == "f32":
        arr[index] = np.nan
    else:
        arr.view(np.uint16)[index] = NAN_BITS[dtype]


_CHUNK = 1 << 22


def normal(rng: np.random.Generator, shape) -> np.ndarray:
    """float32 N(0, 1) draws of `shape` (small tensors only)."""
    return rng.standard_normal(size=shape, dtype=np.float32)


def normal_cast(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) tensor of `shape` in storage dtype `dtype`.

    Up to 4M elements the values come straight from `rng`. Larger tensors are
    filled in 4M-element chunks, chunk i from its own generator seeded by the
    i-th of a list of 64-bit seeds drawn from `rng`, so that the chunks can be
    drawn and cast on several threads with a result that does not depend on
    the thread count.
    """
    n = int(np.prod(shape))
    if n <= _CHUNK:
        return cast(rng.standard_normal(size=shape, dtype=np.float32), dtype)
    out = np.empty(n, dtype=STORAGE[dtype])
    seeds = rng.integers(0, np.iinfo(np.int64).max, size=-(-n // _CHUNK))

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = np.random.default_rng(int(seeds[i])).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = cast(x, dtype)

    from concurrent.futures import ThreadPoolExecutor
    import os
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(len(seeds))))
    return out.reshape(shape)


@dataclass
class PagedCase:
    """One batch of paged-attention inputs.

    k_cache / v_cache are [num_blocks, num_heads, block_size, head_dim].
    block_tables is [num_seqs, max_blocks_per_seq]; entries past a sequence's
    last block hold `pad_entry`.
    For decode, q is [num_seqs, num_heads, head_dim]; for a prefill chunk it is
    [total_queries, num_heads, head_dim] with rows split by cu_q_lens.
    new_seq / new_pos / new_key / new_value describe tokens whose K/V are to be
    written into the cache before attention: token t belongs to sequence
    new_seq[t] at logical position new_pos[t].
    """

    name: str
    dtype: str
    num_heads: int
    head_dim: int
    block_size: int
    context_lens: np.ndarray
    block_tables: np.ndarray
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    scale: float
    seq_blocks: list = field(default_factory=list)  # physical ids per seq, logical order
    cu_q_lens: Optional[np.ndarray] = None
    new_seq: Optional[np.ndarray] = None
    new_pos: Optional[np.ndarray] = None
    new_key: Optional[np.ndarray] = None
    new_value: Optional[np.ndarray] = None
    block_mapping: Optional[np.ndarray] = None  # int64 [pairs, 2] (src, dst)
    pad_entry: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elt_bytes(self) -> int:
        return ELT_BYTES[self.dtype]


def blocks_needed(n: int, block_size: int) -> int:
    """Number of whole blocks that hold n tokens (ceil)."""
    return -(-int(n) // int(block_size))


def kv_bytes_per_token(num_heads: int, head_dim: int, elt_bytes: int, layers: int = 1) -> int:
    """K and V bytes one token occupies in the cache across `layers` layers."""
    return 2 * num_heads * head_dim * elt_bytes * layers


def logical_kv_bytes(context_lens, num_heads: int, head_dim: int, elt_bytes: int) -> int:
    """K+V bytes of the valid tokens of a batch: what attention must read once."""
    return int(np.asarray(context_lens, dtype=np.int64).sum()) * kv_bytes_per_token(
        num_heads, head_dim, elt_bytes)


def _tables(seq_blocks: Sequence[Sequence[int]], width: int, pad: int) -> np.ndarray:
    bt = np.full((len(seq_blocks), width), pad, dtype=np.int32)
    for s, blks in enumerate(seq_blocks):
        bt[s, : len(blks)] = np.asarray(blks, dtype=np.int32)
    return bt


def _fill_pool(rng, num_blocks, H, B, D, dtype):
    k = normal_cast(rng, (num_blocks, H, B, D), dtype)
    v = normal_cast(rng, (num_blocks, H, B, D), dtype)
    return k, v


def make_decode_case(
    num_seqs: int,
    num_heads: int,
    head_dim: int,
    block_size: int,
    dtype: str,
    context_lens: Union[Sequence[int], Callable[[np.random.Generator, int], np.ndarray]],
    seed: int = 0,
    extra_blocks: int = 0,
    max_blocks_per_seq: Optional[int] = None,
    placement: str = "permuted",
    poison_unused: bool = False,
    pad_entry: int = 0,
    new_tokens: bool = False,
    name: str = "custom",
    pool_blocks: Optional[int] = None,
) -> PagedCase:
    """General decode batch.

    context_lens is either an explicit list or a function rng -> lengths.
    The pool has sum(ceil(ctx/B)) + extra_blocks blocks (or pool_blocks). With
    placement "permuted" the blocks are a random permutation of the pool, handed
    out to the sequences in order; with "identity" sequence s gets the next
    consecutive physical ids, so its K/V are contiguous in the pool.
    poison_unused writes NaN into every cache slot that is not a valid token of
    some sequence; pad_entry is written into unused table entries.
    new_tokens draws one new K/V row per sequence for position ctx-1.
    """
    if dtype not in DTYPES:
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    if callable(context_lens):
        ctx = np.asarray(context_lens(rng, num_seqs), dtype=np.int32)
    else:
        ctx = np.asarray(context_lens, dtype=np.int32)
    assert ctx.shape == (num_seqs,)
    nblk = [blocks_needed(n, block_size) for n in ctx]
    used = int(sum(nblk))
    N = pool_blocks if pool_blocks is not None else used + extra_blocks
    assert N >= used
    if placement == "permuted":
        perm = rng.permutation(N)
    elif placement == "identity":
        perm = np.arange(N)
    else:
        raise ValueError(placement)
    seq_blocks, off = [], 0
    for nb in nblk:
        seq_blocks.append([int(x) for x in perm[off : off + nb]])
        off += nb
    M = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, max(nblk) if nblk else 1)
    assert M >= (max(nblk) if nblk else 0)
    q = normal_cast(rng, (num_seqs, num_heads, head_dim), dtype)
    k, v = _fill_pool(rng, N, num_heads, block_size, head_dim, dtype)
    case = PagedCase(
        name=name, dtype=dtype, num_heads=num_heads, head_dim=head_dim,
        block_size=block_size, context_lens=ctx,
        block_tables=_tables(seq_blocks, M, pad_entry), q=q, k_cache=k, v_cache=v,
        scale=1.0 / float(np.sqrt(head_dim)), seq_blocks=seq_blocks, pad_entry=pad_entry,
    )
    if new_tokens:
        case.new_seq = np.arange(num_seqs, dtype=np.int32)
        case.new_pos = (ctx.astype(np.int64) - 1)
        case.new_key = normal_cast(rng, (num_seqs, num_heads, head_dim), dtype)
        case.new_value = normal_cast(rng, (num_seqs, num_heads, head_dim), dtype)
    if poison_unused:
        poison_outside_context(case)
    return case


def valid_slot_mask(case: PagedCase) -> np.ndarray:
    """[num_blocks, block_size] bool: True where a slot holds a valid token.

    Walks each sequence's block list in logical order; the last block of a
    sequence holds ctx - (nblocks-1)*B tokens. Used only to place poison.
    """
    B = case.block_size
    mask = np.zeros((case.num_blocks, B), dtype=bool)
    for s, blks in enumerate(case.seq_blocks):
        remaining = int(case.context_lens[s])
        for phys in blks:
            take = min(B, remaining)
            mask[phys, :take] = True
            remaining -= take
    return mask


def poison_outside_context(case: PagedCase) -> None:
    mask = valid_slot_mask(case)
    for arr in (case.k_cache, case.v_cache):
        nb, sl = np.nonzero(~mask)
        if nb.size:
            view = arr.transpose(0, 2, 1, 3)  # [N, B, H, D] view
            poison(view, case.dtype, (nb, sl))


# ---------------------------------------------------------------------------
# The five named workloads. Seed 0 throughout.
# ---------------------------------------------------------------------------

OPT13B = dict(num_heads=40, head_dim=128, block_size=16)


def tiny_f32(seed: int = 0, poisoned: bool = False) -> PagedCase:
    """4 sequences, 8 heads x 64, B=16, fp32; lengths uniform in [1, 100];
    a 64-block pool handed out from a random permutation."""
    return make_decode_case(
        4, 8, 64, 16, "f32", lambda r, n: r.integers(1, 101, size=n), seed=seed,
        pool_blocks=64, max_blocks_per_seq=7, poison_unused=poisoned,
        pad_entry=-1 if poisoned else 0, new_tokens=False,
        name="tiny_f32" + ("_poisoned" if poisoned else ""))


def _shape(block_size: int) -> dict:
    return dict(OPT13B, block_size=block_size)


def _suffix(block_size: int) -> str:
    return "" if block_size == OPT13B["block_size"] else f"_B{block_size}"


def opt13b_b64(seed: int = 0, dtype: str = "f16", block_size: int = 16, num_seqs: int = 64) -> PagedCase:
    """OPT-13B layer: batch 64 (or num_seqs), 40 heads x 128, B=16 (or
    block_size), lengths uniform in [1, 2048]; the pool holds exactly the
    needed blocks, placed by a random permutation; one new token per
    sequence at position ctx-1."""
    return make_decode_case(
        num_seqs, dtype=dtype, context_lens=lambda r, n: r.integers(1, 2049, size=n), seed=seed,
        max_blocks_per_seq=-(-2048 // block_size), new_tokens=True,
        name=f"opt13b_b{num_seqs}_" + dtype + _suffix(block_size), **_shape(block_size))


def _lognormal_ctx(r, n):
    return np.clip(np.rint(r.lognormal(mean=np.log(300.0), sigma=1.0, size=n)), 8, 2048).astype(np.int32)


def large_batch_b256(seed: int = 0, dtype: str = "f16", block_size: int = 16, num_seqs: int = 256) -> PagedCase:
    """Batch 256 (or num_seqs) with lognormal lengths (median 300, sigma 1,
    clipped to [8, 2048]), random placement; one new token per sequence at
    ctx-1."""
    return make_decode_case(
        num_seqs, dtype=dtype, context_lens=_lognormal_ctx, seed=seed,
        max_blocks_per_seq=-(-2048 // block_size), new_tokens=True,
        name=f"large_batch_b{num_seqs}_" + dtype + _suffix(block_size), **_shape(block_size))


def parallel_sampling(seed: int = 0, prompt_len: int = 512, groups: int = 32, samples: int = 6,
                      dtype: str = "f16", num_heads: int = 40, head_dim: int = 128,
                      block_size: int = 16, max_tail: int = 256) -> PagedCase:
    """Parallel sampling: `groups` prompts of `prompt_len` tokens, each decoded
    by `samples` samples that share the prompt's physical blocks.

    The last prompt block is copy-on-written for samples 1..samples-1 (sample 0,
    the last remaining sharer, keeps the original), so every group contributes
    samples-1 (src, dst) pairs to block_mapping. Divergent tails of 1..max_tail
    tokens live in private blocks. The dst blocks start with random content;
    attention is only meaningful after the copy.
    """
    B = block_size
    rng = np.random.default_rng(seed)
    S = groups * samples
    tails = rng.integers(1, max_tail + 1, size=S).astype(np.int32)
    ctx = (prompt_len + tails).astype(np.int32)
    p_blocks = blocks_needed(prompt_len, B)
    total = [blocks_needed(n, B) for n in ctx]
    private = [t - p_blocks for t in total]
    N = groups * p_blocks + groups * (samples - 1) + int(sum(private))
    perm = rng.permutation(N)
    it = iter(int(x) for x in perm)
    seq_blocks, pairs = [], []
    for g in range(groups):
        prompt = [next(it) for _ in range(p_blocks)]
        copies = [next(it) for _ in range(samples - 1)]
        for k in range(samples):
            s = g * samples + k
            last = prompt[-1] if k == 0 else copies[k - 1]
            seq_blocks.append(prompt[:-1] + [last] + [next(it) for _ in range(private[s])])
        pairs.extend((prompt[-1], c) for c in copies)
    M = blocks_needed(prompt_len + max_tail, B)
    q = normal_cast(rng, (S, num_heads, head_dim), dtype)
    k, v = _fill_pool(rng, N, num_heads, B, head_dim, dtype)
    return PagedCase(
        name=f"parallel_sampling_p{prompt_len}_{dtype}" + _suffix(B), dtype=dtype, num_heads=num_heads,
        head_dim=head_dim, block_size=B, context_lens=ctx, block_tables=_tables(seq_blocks, M, 0),
        q=q, k_cache=k, v_cache=v, scale=1.0 / float(np.sqrt(head_dim)), seq_blocks=seq_blocks,
        block_mapping=np.asarray(pairs, dtype=np.int64).reshape(-1, 2))


def make_prefill_case(num_seqs: int, q_len: int, cached: Union[Sequence[int], Callable], num_heads: int,
                      head_dim: int, block_size: int, dtype: str, seed: int = 0,
                      max_blocks_per_seq: Optional[int] = None, placement: str = "permuted",
                      q_lens: Optional[Sequence[int]] = None, name: str = "prefill") -> PagedCase:
    """Chunked prefill: sequence s has `cached[s]` tokens already in the cache
    and a chunk of q_len (or q_lens[s]) new queries at positions cached[s]..;
    context_lens include the chunk. The chunk's own K/V are drawn as new_key /
    new_value and must be written into the cache before attention."""
    rng = np.random.default_rng(seed)
    c = np.asarray(cached(rng, num_seqs) if callable(cached) else cached, dtype=np.int32)
    ql = np.full(num_seqs, q_len, dtype=np.int32) if q_lens is None else np.asarray(q_lens, np.int32)
    ctx = (c + ql).astype(np.int32)
    nblk = [blocks_needed(n, block_size) for n in ctx]
    N = int(sum(nblk))
    perm = rng.permutation(N) if placement == "permuted" else np.arange(N)
    seq_blocks, off = [], 0
    for nb in nblk:
        seq_blocks.append([int(x) for x in perm[off: off + nb]])
        off += nb
    M = max_blocks_per_seq if max_blocks_per_seq is not None else max(nblk)
    T = int(ql.sum())
    cu = np.zeros(num_seqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    q = normal_cast(rng, (T, num_heads, head_dim), dtype)
    k, v = _fill_pool(rng, N, num_heads, block_size, head_dim, dtype)
    nk = normal_cast(rng, (T, num_heads, head_dim), dtype)
    nv = normal_cast(rng, (T, num_heads, head_dim), dtype)
    new_seq = np.repeat(np.arange(num_seqs, dtype=np.int32), ql)
    new_pos = np.concatenate([np.arange(c[s], ctx[s], dtype=np.int64) for s in range(num_seqs)])
    return PagedCase(
        name=name, dtype=dtype, num_heads=num_heads, head_dim=head_dim, block_size=block_size,
        context_lens=ctx, block_tables=_tables(seq_blocks, M, 0), q=q, k_cache=k, v_cache=v,
        scale=1.0 / float(np.sqrt(head_dim)), seq_blocks=seq_blocks, cu_q_lens=cu,
        new_seq=new_seq, new_pos=new_pos, new_key=nk, new_value=nv)


def chunked_prefill(seed: int = 0, dtype: str = "bf16") -> PagedCase:
    """16 sequences, each a 256-query chunk after 0..1792 cached tokens in
    scattered blocks; 40 heads x 128, B=16, bf16."""
    return make_prefill_case(16, 256, lambda r, n: r.integers(0, 1793, size=n), seed=seed,
                             max_blocks_per_seq=128, dtype=dtype, name="chunked_prefill_" + dtype,
                             **OPT13B)


WORKLOADS = {
    "tiny_f32": tiny_f32,
    "opt13b_b64": opt13b_b64,
    "large_batch_b256": large_batch_b256,
    "parallel_sampling": parallel_sampling,
    "chunked_prefill": chunked_prefill,
}
