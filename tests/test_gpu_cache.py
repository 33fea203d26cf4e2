"""GPU parity of the cache write and the block copy (bit-exact over the whole
pool), and of the full-size workloads that use them: the large batch with
new-token writes and the parallel-sampling batch with copy-on-write."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_109_amd as pa
import workloads as W
from gpu_util import DeviceCase, check_attention, dev, device_slots, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", W.DTYPES)
@pytest.mark.parametrize("D,B", [(64, 4), (128, 16), (128, 32)])
def test_reshape_and_cache_bit_exact(dtype, D, B):
    rng = np.random.default_rng(D + B)
    N, H, T = 37, 5, 50
    k = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), dtype)
    v = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), dtype)
    qkv = W.cast(rng.standard_normal((T, 3, H, D), dtype=np.float32), dtype)   # fused QKV rows
    slots = rng.permutation(N * B)[:T].astype(np.int64)
    slots[::7] = -1
    kd, vd, qkvd = dev(k, dtype), dev(v, dtype), dev(qkv, dtype)
    say(f"  reshape_and_cache {dtype} D={D} B={B} T={T}")
    pa.reshape_and_cache(qkvd[:, 1], qkvd[:, 2], kd, vd, dev(slots))
    torch.cuda.synchronize()
    oracle.reshape_and_cache(k, v, np.ascontiguousarray(qkv[:, 1]), np.ascontiguousarray(qkv[:, 2]), slots, dtype)
    assert host(kd, dtype).tobytes() == k.tobytes()
    assert host(vd, dtype).tobytes() == v.tobytes()


def test_reshape_and_cache_skips_out_of_pool_slots():
    k = torch.zeros(4, 2, 16, 64, dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    key = torch.ones(3, 2, 64, dtype=torch.float16, device="cuda")
    pa.reshape_and_cache(key, key, k, v, torch.tensor([5, 64, 1 << 40], dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert int((k != 0).sum()) == 2 * 64 and bool((k[0, :, 5] == 1).all())


@pytest.mark.parametrize("layers,shape", [(1, (24, 3, 16, 64)), (3, (24, 3, 16, 64)), (70, (24, 3, 16, 64)),
                                          (2, (12, 5, 16, 128)), (1, (16, 40, 16, 128))])
def test_copy_blocks_bit_exact(layers, shape):
    # Blocks of 6 KB (less than one workgroup's 8 KB chunk), 20 KB (two chunks
    # and a partial third) and 160 KB (OPT-13B: twenty whole chunks).
    rng = np.random.default_rng(layers)
    N, H, B, D = shape
    ks = [W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), "bf16") for _ in range(layers)]
    vs = [W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), "bf16") for _ in range(layers)]
    pairs = np.array([[2, 9], [2, 10], [2, 11], [5, 0], [7, 8], [4, 3]], np.int64)
    kd = [dev(a, "bf16") for a in ks]
    vd = [dev(a, "bf16") for a in vs]
    say(f"  copy_blocks layers={layers} shape={shape} pairs={len(pairs)}")
    pa.copy_blocks(kd, vd, dev(pairs))
    torch.cuda.synchronize()
    oracle.copy_blocks(ks, vs, pairs)
    for a, b in zip(kd + vd, ks + vs):
        assert host(a, "bf16").tobytes() == b.tobytes()


def test_copy_blocks_skips_out_of_pool_pairs():
    k = torch.arange(4 * 2 * 4 * 64, dtype=torch.float32, device="cuda").view(4, 2, 4, 64)
    v = k.clone()
    before = k.clone()
    pa.copy_blocks([k], [v], torch.tensor([[0, 4], [9, 1], [1, 2]], dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(k[2], before[1]) and torch.equal(k[[0, 1, 3]], before[[0, 1, 3]])


# ------------------------------------------------------------ full-size workloads

def test_large_batch_b256_full_size():
    """Write the 256 new tokens (position ctx-1) into the cache, then decode."""
    c = W.large_batch_b256()
    dc = DeviceCase(c)
    slots = device_slots(c, dc.block_tables)
    want_slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    assert np.array_equal(slots.cpu().numpy(), want_slots)
    say(f"  large batch: reshape {len(slots)} tokens, then decode")
    pa.reshape_and_cache(dev(c.new_key, c.dtype), dev(c.new_value, c.dtype), dc.k_cache, dc.v_cache, slots)
    torch.cuda.synchronize()
    oracle.reshape_and_cache(c.k_cache, c.v_cache, c.new_key, c.new_value, want_slots, c.dtype)
    assert host(dc.k_cache, c.dtype).tobytes() == c.k_cache.tobytes()
    assert host(dc.v_cache, c.dtype).tobytes() == c.v_cache.tobytes()
    pa.paged_attention_decode(dc.out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                              c.max_context_len, c.scale)
    ref = oracle.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale, c.dtype)
    say("  max err", check_attention(dc.out, ref, c.dtype, c.name))


@pytest.mark.parametrize("prompt_len", [512, 500])
def test_parallel_sampling_full_size(prompt_len):
    """Copy-on-write of each group's last prompt block for 5 of its 6 samples
    (one launch), then decode all 192 samples over shared and private blocks."""
    c = W.parallel_sampling(prompt_len=prompt_len)
    dc = DeviceCase(c)
    say(f"  parallel sampling p={prompt_len}: copy {len(c.block_mapping)} pairs, then decode")
    pa.copy_blocks([dc.k_cache], [dc.v_cache], dev(c.block_mapping))
    torch.cuda.synchronize()
    oracle.copy_blocks([c.k_cache], [c.v_cache], c.block_mapping)
    assert host(dc.k_cache, c.dtype).tobytes() == c.k_cache.tobytes()
    assert host(dc.v_cache, c.dtype).tobytes() == c.v_cache.tobytes()
    pa.paged_attention_decode(dc.out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                              c.max_context_len, c.scale)
    ref = oracle.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale, c.dtype)
    say("  max err", check_attention(dc.out, ref, c.dtype, c.name))


def test_parallel_sampling_copy_across_40_layers():
    """The same 160 pairs over 40 layers in one call: every dst block equals
    its src in every layer and nothing else changes (the copy's definition,
    checked on the device at full size)."""
    c = W.parallel_sampling(groups=32, samples=6, num_heads=40, head_dim=128)
    N = c.num_blocks
    pairs = dev(c.block_mapping)
    g = torch.Generator(device="cuda").manual_seed(0)
    ks = [torch.randint(-30000, 30000, (N, 40, 16, 128), dtype=torch.int16, device="cuda", generator=g)
          .view(torch.float16) for _ in range(40)]
    vs = [torch.randint(-30000, 30000, (N, 40, 16, 128), dtype=torch.int16, device="cuda", generator=g)
          .view(torch.float16) for _ in range(40)]
    src, dst = c.block_mapping[:, 0], c.block_mapping[:, 1]
    keep = np.setdiff1d(np.arange(N), dst)
    keep_t = torch.from_numpy(keep).cuda()
    before = [(a.view(torch.int16)[src].clone(), a.view(torch.int16)[keep_t].clone()) for a in ks + vs]
    say(f"  copy_blocks 40 layers x {len(src)} pairs, pool {N} blocks")
    pa.copy_blocks(ks, vs, pairs)
    torch.cuda.synchronize()
    dst_t = torch.from_numpy(dst).cuda()
    for a, (s_before, keep_before) in zip(ks + vs, before):
        bits = a.view(torch.int16)
        assert torch.equal(bits[dst_t], s_before)
        assert torch.equal(bits[keep_t], keep_before)


@pytest.mark.parametrize("words16,groups", [(1, 1), (1, 8), (259, 7), (65536 + 3, 300), (1 << 20, 2048)])
def test_stream_read_reads_every_word(words16, groups):
    # The XOR of the per-wave sink words is the XOR of every 32-bit word of
    # the buffer exactly when each 16-byte chunk was read once.
    rng = np.random.default_rng(words16 + groups)
    data = rng.integers(0, 2**32, size=4 * words16, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(data.view(np.int32)).cuda()
    sink = torch.zeros(4 * groups, dtype=torch.int32, device="cuda")
    say(f"  stream_read {16 * words16} B, {groups} workgroups")
    pa.stream_read(buf, sink, groups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(data)


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_swap_blocks_out_to_pinned_host_and_back_bit_exact(dtype):
    """Blocks of every layer's K and V go from the device pool to a pinned
    host pool and back to other device blocks; both whole pools must equal
    the oracle's byte for byte (so nothing else was written)."""
    rng = np.random.default_rng(31)
    Nd, Nh, L, H, B, D = 40, 12, 2, 3, 16, 64
    dev_np = [W.cast(rng.standard_normal((Nd, H, B, D), dtype=np.float32), dtype) for _ in range(2 * L)]
    host_np = [W.cast(rng.standard_normal((Nh, H, B, D), dtype=np.float32), dtype) for _ in range(2 * L)]
    dev_t = [dev(a, dtype) for a in dev_np]
    def pinned(a):
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if dtype == "bf16" else a))
        return (t.view(torch.bfloat16) if dtype == "bf16" else t).pin_memory()

    host_t = [pinned(a) for a in host_np]
    assert all(t.is_pinned() for t in host_t)
    out_map = np.stack([rng.choice(Nd, 9, replace=False), rng.choice(Nh, 9, replace=False)], axis=1)
    say(f"  swap out {dtype}: {len(out_map)} blocks x {2 * L} caches to pinned host memory")
    pa.swap_blocks(dev_t, host_t, dev(out_map.astype(np.int64)))
    torch.cuda.synchronize()
    oracle.swap_blocks(dev_np, host_np, out_map)
    for t, a in zip(host_t, host_np):
        assert host(t, dtype).tobytes() == a.tobytes()
    in_map = np.stack([out_map[:, 1], rng.choice(Nd, 9, replace=False)], axis=1).astype(np.int64)
    in_map_pinned = torch.from_numpy(in_map).pin_memory()
    say(f"  swap in {dtype}: mapping in pinned host memory")
    pa.swap_blocks(host_t, dev_t, in_map_pinned)
    torch.cuda.synchronize()
    oracle.swap_blocks(host_np, dev_np, in_map)
    for t, a in zip(dev_t, dev_np):
        assert host(t, dtype).tobytes() == a.tobytes()


def test_swap_blocks_refuses_pageable_host_memory():
    # The mapping's source index is outside the pool, so even a launch
    # would touch no cache block; the call must refuse before launching.
    src = torch.zeros(4, 2, 16, 64, dtype=torch.float16)  # ordinary (pageable) host memory
    dst = torch.zeros(4, 2, 16, 64, dtype=torch.float16, device="cuda")
    mapping = torch.tensor([[1 << 40, 0]], dtype=torch.int64, device="cuda")
    with pytest.raises(pa.PagedAttnError) as e:
        pa.swap_blocks([src], [dst], mapping)
    assert e.value.status == 1 and "pinned" in str(e.value)
