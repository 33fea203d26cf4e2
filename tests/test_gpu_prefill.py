"""GPU parity of chunked-prefill paged attention (MFMA) against the CPU oracle.

Each case first writes the chunk's own K/V into the cache with
reshape_and_cache (slots from the library's device translation, checked
against the oracle's), then runs the causal chunk attention and compares every output
element with oracle.prefill_chunk to the fp16/bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_109_amd as pa
import workloads as W
from gpu_util import DeviceCase, as_f64, check_attention, dev, device_slots, host, plant_value, say

pytestmark = pytest.mark.gpu


def run_prefill(c, poison=False):
    if poison:
        W.poison_outside_context(c)
    dc = DeviceCase(c)
    slots = device_slots(c, dc.block_tables)
    want_slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    assert np.array_equal(slots.cpu().numpy(), want_slots)
    say(f"  prefill {c.name}: S={c.num_seqs} H={c.num_heads} B={c.block_size} {c.dtype} q_lens="
        f"{list(np.diff(c.cu_q_lens))[:6]} ctx={list(c.context_lens)[:6]}")
    pa.reshape_and_cache(dev(c.new_key, c.dtype), dev(c.new_value, c.dtype), dc.k_cache, dc.v_cache, slots)
    out = torch.empty_like(dc.q)
    max_q = int(np.diff(c.cu_q_lens).max())
    pa.paged_attention_prefill_chunk(out, dc.q, dev(c.cu_q_lens), dc.k_cache, dc.v_cache, dc.block_tables,
                                     dc.context_lens, max_q, c.max_context_len, c.scale)
    torch.cuda.synchronize()
    oracle.reshape_and_cache(c.k_cache, c.v_cache, c.new_key, c.new_value, want_slots, c.dtype)
    assert host(dc.k_cache, c.dtype).tobytes() == c.k_cache.tobytes()
    ref = oracle.prefill_chunk(c.q, c.cu_q_lens, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale,
                               c.dtype)
    return out, ref


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B", [4, 8, 16, 32, 64])
def test_prefill_shapes(dtype, B):
    c = W.make_prefill_case(4, 0, [0, 37, 300, 5], 3, 128, B, dtype, seed=B, q_lens=[5, 130, 256, 1],
                            name=f"prefill_B{B}")
    out, ref = run_prefill(c)
    say("  max err", check_attention(out, ref, dtype, c.name))


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("f32", 64), ("f16", 64), ("bf16", 64)])
@pytest.mark.parametrize("B", [4, 16, 64])
def test_prefill_general_shapes(dtype, D, B):
    """fp32 and head_dim 64 run on the vector-ALU prefill kernel (8 queries
    per wave): ragged chunks (1, 5, 9, 130 queries) after 0..300 cached
    tokens, one chunk longer than its 8-query groups by one."""
    c = W.make_prefill_case(4, 0, [0, 37, 300, 5], 3, D, B, dtype, seed=B + D, q_lens=[5, 130, 9, 1],
                            name=f"prefill_general_{dtype}_D{D}_B{B}")
    out, ref = run_prefill(c)
    say("  max err", check_attention(out, ref, dtype, c.name))


def test_prefill_general_poisoned_slots_are_never_read():
    c = W.make_prefill_case(3, 0, [17, 0, 64], 2, 64, 16, "f16", seed=9, q_lens=[40, 33, 17], name="poison64")
    out, ref = run_prefill(c, poison=True)
    assert not torch.isnan(out).any()
    check_attention(out, ref, "f16", "poisoned, head_dim 64")


def test_prefill_poisoned_slots_are_never_read():
    c = W.make_prefill_case(3, 0, [17, 0, 64], 2, 128, 16, "bf16", seed=5, q_lens=[40, 33, 128], name="poison")
    # Poison everything outside the final contexts; the chunk tokens are written
    # by reshape_and_cache before attention, so they are not poisoned for long.
    out, ref = run_prefill(c, poison=True)
    assert torch.isfinite(out).all()
    check_attention(out, ref, "bf16", "poisoned")


def test_prefill_bf16_values_beyond_f16_range():
    """The P V product runs in f16, so bf16 V values past f16's range (a
    cached token and a chunk token) leave the waves that read them with
    non-finite sums; those waves recompute their queries exactly."""
    c = W.make_prefill_case(3, 0, [40, 0, 200], 2, 128, 16, "bf16", seed=21, q_lens=[100, 64, 150], name="huge")
    plant_value(c, 0, 10, 1, [0, 1, 2, 3], [1e5, -3e6, 1e30, 7e4])
    plant_value(c, 2, 230, 0, [5], [2e5])
    out, ref = run_prefill(c)
    assert torch.isfinite(out).all()
    say("  max err", check_attention(out, ref, "bf16", "V beyond f16's range"))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_nan_value_reaches_only_queries_that_see_it(dtype):
    """A NaN in one V element of a chunk token: exactly the queries at or
    past that position (that head, that dimension) come out NaN, as in the
    oracle; the earlier queries of the same wave, whose weights for it are
    0, stay exact."""
    c = W.make_prefill_case(2, 0, [30, 5], 2, 128, 16, dtype, seed=22, q_lens=[90, 40], name="nan")
    plant_value(c, 0, 70, 1, [7])
    out, ref = run_prefill(c)
    g, r = as_f64(out), ref
    want = np.zeros(r.shape, bool)
    want[int(c.cu_q_lens[0]) + 70 - 30: int(c.cu_q_lens[1]), 1, 7] = True
    assert np.array_equal(np.isnan(r), want)
    assert np.array_equal(np.isnan(g), want)
    out[torch.from_numpy(want).to(out.device)] = 0
    say("  max err", check_attention(out, np.where(want, 0.0, r), dtype, "NaN in one V element"))


def test_single_query_chunk_equals_decode():
    """A one-query chunk is a decode step: both kernels, same inputs."""
    c = W.make_prefill_case(5, 1, [0, 15, 16, 700, 2047], 4, 128, 16, "f16", seed=6, name="q1")
    out, ref = run_prefill(c)
    check_attention(out, ref, "f16", "q1 vs oracle")
    dc = DeviceCase(c)
    slots = device_slots(c, dc.block_tables)
    pa.reshape_and_cache(dev(c.new_key, "f16"), dev(c.new_value, "f16"), dc.k_cache, dc.v_cache, slots)
    pa.paged_attention_decode(dc.out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                              c.max_context_len, c.scale)
    torch.cuda.synchronize()
    check_attention(dc.out, ref, "f16", "q1 decode vs oracle")


def test_chunked_prefill_full_size():
    """16 sequences x 256-query causal chunks over 0..1792 cached tokens,
    40 heads x 128, B=16, bf16 -- every output element against the oracle."""
    c = W.chunked_prefill()
    out, ref = run_prefill(c)
    say("  max err", check_attention(out, ref, "bf16", c.name))


def test_prefill_long_context_small_blocks():
    """A 16,600-token context at B=4: over 4,000 table entries, each 4-row
    load of a 32-key block on its own block."""
    c = W.make_prefill_case(2, 0, [16600, 3], 2, 128, 4, "bf16", seed=11, q_lens=[40, 7], name="long_table")
    out, ref = run_prefill(c)
    say("  max err", check_attention(out, ref, "bf16", c.name))


def test_prefill_three_query_tiles():
    """q_len 300 spans three 128-query tiles; 129 spans two with one query in
    the second."""
    c = W.make_prefill_case(2, 0, [1000, 0], 3, 128, 16, "f16", seed=12, q_lens=[300, 129], name="tiles")
    out, ref = run_prefill(c)
    say("  max err", check_attention(out, ref, "f16", c.name))


@pytest.mark.parametrize("seed", range(8))
def test_random_mfma_chunks(seed):
    """Seeded MFMA shapes: 1-8 sequences x 1-8 heads, chunks of 1 to 384
    queries (one to four 128-query tiles, on and off the tile edges) after
    0-3000 cached tokens, any block size, NaN in every slot outside a
    context."""
    rng = np.random.default_rng(3000 + seed)
    S, H = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    dtype = str(rng.choice(["f16", "bf16"]))
    B = int(rng.choice([4, 8, 16, 32, 64]))
    cached = [int(x) for x in rng.integers(0, 3001, size=S)]
    cached[0] -= cached[0] % B  # one chunk starts on a block boundary
    q_lens = [int(x) for x in rng.choice([1, 16, 63, 64, 65, 127, 128, 129, 255, 256, 300, 384], size=S)]
    c = W.make_prefill_case(S, 0, cached, H, 128, B, dtype, seed=seed, q_lens=q_lens, name=f"mfma_{seed}")
    out, ref = run_prefill(c, poison=True)
    say("  max err", check_attention(out, ref, dtype, c.name))


def test_permuting_physical_blocks_is_bit_identical():
    """The same logical K/V in another physical placement gives the same
    output bytes: the kernel's arithmetic follows logical positions only."""
    c = W.make_prefill_case(3, 0, [100, 1000, 37], 4, 128, 16, "bf16", seed=21, q_lens=[200, 64, 129], name="perm")
    slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    oracle.reshape_and_cache(c.k_cache, c.v_cache, c.new_key, c.new_value, slots, c.dtype)
    perm = np.random.default_rng(2).permutation(c.num_blocks)
    k2 = np.empty_like(c.k_cache)
    k2[perm] = c.k_cache
    v2 = np.empty_like(c.v_cache)
    v2[perm] = c.v_cache
    bt2 = c.block_tables.copy()
    for s, blks in enumerate(c.seq_blocks):
        bt2[s, :len(blks)] = perm[np.asarray(blks)]
    outs = []
    for k, v, bt in ((c.k_cache, c.v_cache, c.block_tables), (k2, v2, bt2)):
        out = torch.empty_like(dev(c.q, "bf16"))
        pa.paged_attention_prefill_chunk(out, dev(c.q, "bf16"), dev(c.cu_q_lens), dev(k, "bf16"), dev(v, "bf16"),
                                         dev(bt), dev(c.context_lens), 200, c.max_context_len, c.scale)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16))
    assert torch.equal(outs[0], outs[1])
