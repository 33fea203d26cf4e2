"""Pools past 4 GiB: every kernel forms 64-bit byte offsets into the caches.

Each cache here holds 140,000 blocks of 8 heads x 16 x 128 fp16/bf16 (4.6 GB),
and the batch's blocks sit at the top of the pool, above the 4 GiB line; the
rest of the pool is left uninitialised. A block's placement changes no
arithmetic, so the outputs must be bit-identical to the same batch in a
compact pool (which is itself checked against the oracle), and writes and
copies must land on exactly the bytes they should.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_109_amd as pa
import workloads as W
from gpu_util import TORCH_DT, check_attention, dev, host, say

pytestmark = pytest.mark.gpu

N_BIG = 140_000  # blocks: 140,000 x 32 KB = 4.59 GB per cache


def place_high(c, dtype):
    """Device caches of N_BIG blocks with the case's blocks at the top of the
    pool (block b of the case at id N_BIG - num_blocks + b), and the tables
    remapped to them."""
    H, B, D = c.num_heads, c.block_size, c.head_dim
    assert H * B * D * 2 * (N_BIG - c.num_blocks) > (1 << 32)  # every used block starts past 4 GiB
    ids = np.arange(c.num_blocks, dtype=np.int64) + (N_BIG - c.num_blocks)
    kd = torch.empty((N_BIG, H, B, D), dtype=TORCH_DT[dtype], device="cuda")
    vd = torch.empty_like(kd)
    idx = torch.from_numpy(ids).cuda()
    kd[idx] = dev(c.k_cache, dtype)
    vd[idx] = dev(c.v_cache, dtype)
    tables = np.where(c.block_tables >= 0, ids[np.clip(c.block_tables, 0, c.num_blocks - 1)], c.block_tables)
    return kd, vd, tables.astype(np.int32), ids


def test_decode_past_4gib():
    c = W.make_decode_case(4, 8, 128, 16, "f16", [300, 1000, 17, 2048], seed=31, max_blocks_per_seq=128)
    ref = oracle.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale, "f16")
    small = pa.paged_attention_decode(torch.empty_like(dev(c.q)), dev(c.q), dev(c.k_cache), dev(c.v_cache),
                                      dev(c.block_tables), dev(c.context_lens), c.max_context_len, c.scale)
    kd, vd, tables, _ = place_high(c, "f16")
    say(f"  decode over a pool of {N_BIG} blocks ({kd.numel() * 2 / 1e9:.2f} GB per cache)")
    big = pa.paged_attention_decode(torch.empty_like(dev(c.q)), dev(c.q), kd, vd, dev(tables), dev(c.context_lens),
                                    c.max_context_len, c.scale)
    torch.cuda.synchronize()
    check_attention(small, ref, "f16", "compact pool")
    assert torch.equal(big.view(torch.int16), small.view(torch.int16))


def test_prefill_past_4gib():
    c = W.make_prefill_case(2, 0, [700, 40], 8, 128, 16, "bf16", seed=32, q_lens=[130, 64], name="big_pool")
    slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    oracle.reshape_and_cache(c.k_cache, c.v_cache, c.new_key, c.new_value, slots, "bf16")
    ref = oracle.prefill_chunk(c.q, c.cu_q_lens, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale,
                               "bf16")
    q = dev(c.q, "bf16")

    def run(k, v, tables):
        out = torch.empty_like(q)
        pa.paged_attention_prefill_chunk(out, q, dev(c.cu_q_lens), k, v, dev(tables), dev(c.context_lens), 130,
                                         c.max_context_len, c.scale)
        torch.cuda.synchronize()
        return out

    small = run(dev(c.k_cache, "bf16"), dev(c.v_cache, "bf16"), c.block_tables)
    kd, vd, tables, _ = place_high(c, "bf16")
    big = run(kd, vd, tables)
    check_attention(small, ref, "bf16", "compact pool")
    assert torch.equal(big.view(torch.int16), small.view(torch.int16))


def test_cache_write_and_copy_past_4gib():
    c = W.make_decode_case(3, 8, 128, 16, "f16", [20, 33, 5], seed=33, max_blocks_per_seq=4)
    kd, vd, tables, ids = place_high(c, "f16")
    # Write one new token per sequence at position ctx (its next slot) and
    # check the rows it lands in.
    rng = np.random.default_rng(5)
    key = W.cast(rng.standard_normal((3, 8, 128), dtype=np.float32), "f16")
    val = W.cast(rng.standard_normal((3, 8, 128), dtype=np.float32), "f16")
    pos = c.context_lens.astype(np.int64)
    assert all(p // 16 < len(b) for p, b in zip(pos, c.seq_blocks))
    slots = np.array([tables[s, p // 16] * 16 + p % 16 for s, p in enumerate(pos)], np.int64)
    pa.reshape_and_cache(dev(key), dev(val), kd, vd, dev(slots))
    # Copy the top block of the pool onto two unused ones, one above and one
    # below 4 GiB.
    top, high = int(ids[-1]), int(ids[0]) - 1
    assert high * 8 * 16 * 128 * 2 > (1 << 32)
    pairs = np.array([[top, high], [top, 5]], np.int64)
    pa.copy_blocks([kd], [vd], dev(pairs))
    torch.cuda.synchronize()
    for s in range(3):
        blk, off = int(slots[s] // 16), int(slots[s] % 16)
        assert host(kd[blk, :, off], "f16").tobytes() == key[s].tobytes()
        assert host(vd[blk, :, off], "f16").tobytes() == val[s].tobytes()
    for dst in (high, 5):
        assert torch.equal(kd[dst], kd[top]) and torch.equal(vd[dst], vd[top])


def test_swap_past_4gib():
    c = W.make_decode_case(2, 8, 128, 16, "f16", [40, 70], seed=34)
    kd, vd, _, ids = place_high(c, "f16")
    # Swap the case's blocks (all past 4 GiB) out to a pinned host pool in
    # reverse order, then back in onto other blocks past 4 GiB.
    n = c.num_blocks
    hk = torch.zeros((n, 8, 16, 128), dtype=torch.float16, pin_memory=True)
    hv = torch.zeros_like(hk, pin_memory=True)
    out_pairs = np.stack([ids, np.arange(n)[::-1]], axis=1).astype(np.int64)
    pa.swap_blocks([kd, vd], [hk, hv], dev(out_pairs))
    torch.cuda.synchronize()
    for i, b in enumerate(ids):
        assert host(hk[n - 1 - i], "f16").tobytes() == c.k_cache[i].tobytes()
        assert host(hv[n - 1 - i], "f16").tobytes() == c.v_cache[i].tobytes()
    back = ids - n  # the n blocks below the case's, still past 4 GiB
    assert int(back[0]) * 8 * 16 * 128 * 2 > (1 << 32)
    in_pairs = np.stack([np.arange(n)[::-1], back], axis=1).astype(np.int64)
    pa.swap_blocks([hk, hv], [kd, vd], dev(in_pairs))
    torch.cuda.synchronize()
    idx = torch.from_numpy(back).cuda()
    assert torch.equal(kd[idx], kd[torch.from_numpy(ids).cuda()])
    assert torch.equal(vd[idx], vd[torch.from_numpy(ids).cuda()])
