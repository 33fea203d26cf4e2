"""The fused cache append + decode (pa_paged_attention_decode_append).

A decode step stores the new token's K/V at position n - 1 and attends over
a context that includes it (the write and the attention of one decode step
in "KV 캐시 관리와 PagedAttention", section on attention over scattered KV).
Every case here runs both ways on identical copies of the pool:
reshape_and_cache at the token's slot followed by paged_attention_decode,
and the fused call. The caches and the outputs must agree byte for byte;
the fused output is also checked against the oracle (its cache write
against the oracle's, bit for bit, and its attention within the attention
tolerance).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_109_amd as pa
import workloads as W
from gpu_util import TORCH_DT, check_attention, dev, host, say

pytestmark = pytest.mark.gpu


def new_token_slots(tables: np.ndarray, ctx: np.ndarray, block_size: int, num_blocks: int) -> np.ndarray:
    """Slot of position n - 1 of every sequence; -1 where n = 0 or the table
    entry is outside the pool (both paths then write nothing)."""
    out = np.full(len(ctx), -1, np.int64)
    for s, n in enumerate(ctx):
        if n >= 1:
            e = int(tables[s, (n - 1) // block_size])
            if 0 <= e < num_blocks:
                out[s] = e * block_size + (n - 1) % block_size
    return out


def new_rows(rng, S, H, D, dtype):
    return W.normal_cast(rng, (S, H, D), dtype), W.normal_cast(rng, (S, H, D), dtype)


def run_both(c, key, value, split_workers=0, key_dev=None, value_dev=None, poison_slot=False, split_call=False):
    """Returns (out_fused, k_fused, v_fused, out_separate, k_sep, v_sep, slots)."""
    dt = c.dtype
    S, H, D, B = c.num_seqs, c.num_heads, c.head_dim, c.block_size
    slots = new_token_slots(c.block_tables, c.context_lens, B, c.num_blocks)
    q, bt, ctx = dev(c.q, dt), dev(c.block_tables), dev(c.context_lens)
    kd = key_dev if key_dev is not None else dev(key, dt)
    vd = value_dev if value_dev is not None else dev(value, dt)
    max_ctx = max(c.max_context_len, 1)

    k_sep, v_sep = dev(c.k_cache, dt), dev(c.v_cache, dt)
    pa.reshape_and_cache(kd, vd, k_sep, v_sep, dev(slots))
    out_sep = pa.paged_attention_decode(torch.empty_like(q), q, k_sep, v_sep, bt, ctx, max_ctx, c.scale,
                                        split_workers=split_workers)

    k_f, v_f = dev(c.k_cache, dt), dev(c.v_cache, dt)
    if poison_slot:  # a stale NaN in the slot being written: never read
        for sl in slots[slots >= 0]:
            k_f[int(sl) // B, :, int(sl) % B] = float("nan")
            v_f[int(sl) // B, :, int(sl) % B] = float("nan")
    out_f = torch.empty_like(q)
    if split_call:
        ws = pa.alloc_decode_workspace(S, H, D, max_ctx, B, split_workers)
        k0, v0 = k_f.clone(), v_f.clone()
        pa.paged_attention_decode_append_partitions(out_f, q, kd, vd, k_f, v_f, bt, ctx, max_ctx, c.scale,
                                                    workspace=ws, split_workers=split_workers)
        torch.cuda.synchronize()
        # The partition pass only reads: the caches are untouched until the reduce.
        assert same_bytes(k_f, k0) and same_bytes(v_f, v0)
        pa.paged_attention_decode_append_reduce(out_f, q, kd, vd, k_f, v_f, bt, ctx, max_ctx, c.scale,
                                                workspace=ws, split_workers=split_workers)
    else:
        pa.paged_attention_decode_append(out_f, q, kd, vd, k_f, v_f, bt, ctx, max_ctx, c.scale,
                                         split_workers=split_workers)
    torch.cuda.synchronize()
    return out_f, k_f, v_f, out_sep, k_sep, v_sep, slots


def same_bytes(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def check_case(c, key, value, what, **kw):
    out_f, k_f, v_f, out_s, k_s, v_s, slots = run_both(c, key, value, **kw)
    assert same_bytes(k_f, k_s) and same_bytes(v_f, v_s), f"{what}: caches differ from the separate write"
    assert same_bytes(out_f, out_s), f"{what}: output differs from reshape_and_cache + decode"
    # The oracle: its cache write, then its decode over the written cache.
    k_ref, v_ref = c.k_cache.copy(), c.v_cache.copy()
    oracle.reshape_and_cache(k_ref, v_ref, key, value, slots, c.dtype)
    assert host(k_f, c.dtype).tobytes() == k_ref.tobytes() and host(v_f, c.dtype).tobytes() == v_ref.tobytes()
    ref = oracle.decode(c.q, k_ref, v_ref, c.block_tables, c.context_lens, c.scale, c.dtype)
    err = check_attention(out_f, ref, c.dtype, what)
    say(f"  {what}: bit-identical to the separate path; vs oracle max_abs {err[0]:.2e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D,B", [(128, 16), (64, 4), (128, 32), (64, 64)])
def test_append_shapes(dtype, D, B):
    lens = [1, 15, 16, 17, 33, 300, 1000, 64]
    c = W.make_decode_case(len(lens), 4, D, B, dtype, lens, seed=D + B, extra_blocks=5,
                           max_blocks_per_seq=-(-1000 // B) + 1)
    key, value = new_rows(np.random.default_rng(B), c.num_seqs, 4, D, dtype)
    check_case(c, key, value, f"{dtype} D={D} B={B}")


@pytest.mark.parametrize("split_workers", [1, 3, 64, 300, 4096])
def test_append_any_split(split_workers):
    c = W.make_decode_case(6, 8, 128, 16, "f16", [5, 160, 161, 1, 700, 48], seed=7, max_blocks_per_seq=48)
    key, value = new_rows(np.random.default_rng(1), 6, 8, 128, "f16")
    check_case(c, key, value, f"split {split_workers}", split_workers=split_workers)


@pytest.mark.parametrize("split_workers", [1, 200, 0])
def test_append_partitions_then_reduce(split_workers):
    c = W.make_decode_case(5, 8, 128, 16, "bf16", [100, 2048, 31, 512, 7], seed=8, max_blocks_per_seq=128)
    key, value = new_rows(np.random.default_rng(2), 5, 8, 128, "bf16")
    check_case(c, key, value, "two calls", split_call=True, split_workers=split_workers)


@pytest.mark.parametrize("split_workers", [0, 1])
def test_append_more_rows_than_one_pass_of_the_store_grid(split_workers):
    # 900 sequences x 40 heads of head_dim 128 (f16) make 1,152,000 16-byte
    # chunks of new rows, more than the reduce's store workgroups cover in one
    # pass (4096 x 256 threads), so its grid-stride loop runs; at one worker
    # no pair is cut and every workgroup of the reduce stores.
    S = 900
    lens = np.random.default_rng(13).integers(1, 40, S).tolist()
    c = W.make_decode_case(S, 40, 128, 16, "f16", lens, seed=13, max_blocks_per_seq=3)
    key, value = new_rows(np.random.default_rng(14), S, 40, 128, "f16")
    check_case(c, key, value, f"{S} sequences, split {split_workers}", split_workers=split_workers)


def test_append_never_reads_the_stale_slot():
    c = W.make_decode_case(4, 4, 128, 16, "f16", [1, 16, 17, 250], seed=9, max_blocks_per_seq=16)
    key, value = new_rows(np.random.default_rng(3), 4, 4, 128, "f16")
    out_f, k_f, v_f, out_s, k_s, v_s, _ = run_both(c, key, value, poison_slot=True)
    assert not torch.isnan(out_f.float()).any()
    assert same_bytes(out_f, out_s) and same_bytes(k_f, k_s) and same_bytes(v_f, v_s)


def test_append_empty_context():
    c = W.make_decode_case(4, 4, 64, 16, "f16", [0, 40, 0, 33], seed=10, extra_blocks=2, max_blocks_per_seq=4)
    key, value = new_rows(np.random.default_rng(4), 4, 4, 64, "f16")
    check_case(c, key, value, "n = 0")


def test_append_out_of_pool_entry_is_neither_read_nor_written():
    # An entry outside the pool inside the context breaks a precondition (the
    # oracle refuses it); the kernels mask that token, and the fused call must
    # then do exactly what the separate path does: write nothing for it.
    c = W.make_decode_case(3, 4, 128, 16, "f16", [40, 17, 33], seed=12, extra_blocks=2, max_blocks_per_seq=4)
    c.block_tables[1, 1] = c.num_blocks + 3  # position 16, the newest token of the 17-token context
    key, value = new_rows(np.random.default_rng(6), 3, 4, 128, "f16")
    out_f, k_f, v_f, out_s, k_s, v_s, slots = run_both(c, key, value)
    assert slots[1] == -1
    assert same_bytes(out_f, out_s) and same_bytes(k_f, k_s) and same_bytes(v_f, v_s)
    k_ref = c.k_cache.copy()
    oracle.reshape_and_cache(k_ref, c.v_cache.copy(), key, value, slots, "f16")
    assert host(k_f, "f16").tobytes() == k_ref.tobytes()


def test_append_fused_qkv_strides():
    c = W.make_decode_case(5, 8, 128, 16, "bf16", [9, 400, 33, 16, 1], seed=11, max_blocks_per_seq=32)
    rng = np.random.default_rng(5)
    qkv = W.normal_cast(rng, (5, 3, 8, 128), "bf16")
    qkv_dev = dev(qkv, "bf16")
    key, value = np.ascontiguousarray(qkv[:, 1]), np.ascontiguousarray(qkv[:, 2])
    check_case(c, key, value, "fused QKV slices", key_dev=qkv_dev[:, 1], value_dev=qkv_dev[:, 2])


def test_append_opt13b_b64_full_size():
    c = W.opt13b_b64()
    assert c.new_key is not None and (c.new_pos == c.context_lens - 1).all()
    out_f, k_f, v_f, out_s, k_s, v_s, slots = run_both(c, c.new_key, c.new_value)
    assert same_bytes(out_f, out_s) and same_bytes(k_f, k_s) and same_bytes(v_f, v_s)
    # The written rows, against the oracle's write, and a sample of outputs
    # against the oracle's decode over the written cache.
    k_ref, v_ref = c.k_cache.copy(), c.v_cache.copy()
    oracle.reshape_and_cache(k_ref, v_ref, c.new_key, c.new_value, slots, c.dtype)
    rows = [(int(s) // 16, int(s) % 16) for s in slots]
    for blk, off in rows:
        assert host(k_f[blk, :, off], "f16").tobytes() == k_ref[blk, :, off].tobytes()
        assert host(v_f[blk, :, off], "f16").tobytes() == v_ref[blk, :, off].tobytes()
    pick = np.array([0, 17, 40, 63])
    ref = oracle.decode(c.q[pick], k_ref, v_ref, c.block_tables[pick], c.context_lens[pick], c.scale, "f16")
    err = check_attention(out_f[torch.from_numpy(pick).cuda()], ref, "f16", "opt13b_b64 sample")
    say(f"  opt13b_b64: fused = separate, bit for bit; sampled vs oracle max_abs {err[0]:.2e}")
