"""The fused chunk write + prefill (pa_paged_attention_prefill_chunk_append).

A chunk's own K/V are stored and then attended over (the cache write of the
review's section 5.1 followed by chunked prefill). Every case runs both ways
on identical copies of the pool: reshape_and_cache at the chunk's slots
followed by paged_attention_prefill_chunk, and the fused call. Caches and
outputs must agree byte for byte; the fused result is also checked against
the oracle (its cache write bit for bit, its attention within the attention
tolerance).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_109_amd as pa
import workloads as W
from gpu_util import check_attention, dev, host, plant_value, say

pytestmark = pytest.mark.gpu


def same_bytes(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def run_both(c, key_dev=None, value_dev=None):
    dt = c.dtype
    slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    q, cu, bt, ctx = dev(c.q, dt), dev(c.cu_q_lens), dev(c.block_tables), dev(c.context_lens)
    nk = key_dev if key_dev is not None else dev(c.new_key, dt)
    nv = value_dev if value_dev is not None else dev(c.new_value, dt)
    max_q = int(np.diff(c.cu_q_lens).max())
    k_s, v_s = dev(c.k_cache, dt), dev(c.v_cache, dt)
    pa.reshape_and_cache(nk, nv, k_s, v_s, dev(slots))
    out_s = pa.paged_attention_prefill_chunk(torch.empty_like(q), q, cu, k_s, v_s, bt, ctx, max_q,
                                             c.max_context_len, c.scale)
    k_f, v_f = dev(c.k_cache, dt), dev(c.v_cache, dt)
    out_f = pa.paged_attention_prefill_chunk_append(torch.empty_like(q), q, nk, nv, cu, k_f, v_f, bt, ctx, max_q,
                                                    c.max_context_len, c.scale)
    torch.cuda.synchronize()
    return out_f, k_f, v_f, out_s, k_s, v_s, slots


def check_case(c, what, **kw):
    out_f, k_f, v_f, out_s, k_s, v_s, slots = run_both(c, **kw)
    assert same_bytes(k_f, k_s) and same_bytes(v_f, v_s), f"{what}: caches differ from the separate write"
    assert same_bytes(out_f, out_s), f"{what}: output differs from reshape_and_cache + prefill"
    k_ref, v_ref = c.k_cache.copy(), c.v_cache.copy()
    oracle.reshape_and_cache(k_ref, v_ref, c.new_key, c.new_value, slots, c.dtype)
    assert host(k_f, c.dtype).tobytes() == k_ref.tobytes() and host(v_f, c.dtype).tobytes() == v_ref.tobytes()
    ref = oracle.prefill_chunk(c.q, c.cu_q_lens, k_ref, v_ref, c.block_tables, c.context_lens, c.scale, c.dtype)
    err = check_attention(out_f, ref, c.dtype, what)
    say(f"  {what}: bit-identical to the separate path; vs oracle max_abs {err[0]:.2e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B", [4, 8, 16, 32, 64])
def test_prefill_append_shapes(dtype, B):
    c = W.make_prefill_case(4, 0, [0, 37, 700, 1500], 4, 128, B, dtype, seed=40 + B, q_lens=[1, 5, 130, 256],
                            name="append")
    check_case(c, f"{dtype} B={B}")


def test_prefill_append_more_than_64_sequences():
    # Past 64 sequences the kernel schedules the query tiles without ranking
    # them by context length.
    c = W.make_prefill_case(70, 0, lambda r, n: r.integers(0, 300, n), 2, 128, 16, "bf16", seed=49,
                            q_lens=np.random.default_rng(50).integers(1, 40, 70), name="many")
    check_case(c, "70 sequences")


def test_prefill_append_three_query_tiles():
    c = W.make_prefill_case(2, 0, [100, 3], 8, 128, 16, "bf16", seed=44, q_lens=[300, 257], name="tiles")
    check_case(c, "three query tiles")


def test_prefill_append_fused_qkv_strides():
    c = W.make_prefill_case(3, 0, [20, 400, 0], 8, 128, 16, "f16", seed=45, q_lens=[64, 17, 200], name="qkv")
    T = int(c.cu_q_lens[-1])
    rng = np.random.default_rng(46)
    qkv = W.normal_cast(rng, (T, 3, 8, 128), "f16")
    c.new_key, c.new_value = np.ascontiguousarray(qkv[:, 1]), np.ascontiguousarray(qkv[:, 2])
    qkv_d = dev(qkv, "f16")
    check_case(c, "fused QKV slices", key_dev=qkv_d[:, 1], value_dev=qkv_d[:, 2])


def test_prefill_append_chunked_prefill_full_size():
    c = W.chunked_prefill()
    out_f, k_f, v_f, out_s, k_s, v_s, _ = run_both(c)
    assert same_bytes(out_f, out_s) and same_bytes(k_f, k_s) and same_bytes(v_f, v_s)
    say("  chunked_prefill: fused = separate, bit for bit (output and both caches)")


def test_prefill_append_bf16_values_beyond_f16_range():
    # The waves that read them recompute their queries from the new rows
    # (chunk tokens) and the cache (cached tokens).
    c = W.make_prefill_case(3, 0, [40, 0, 200], 2, 128, 16, "bf16", seed=23, q_lens=[100, 64, 150], name="huge")
    plant_value(c, 0, 10, 1, [0, 1, 2, 3], [1e5, -3e6, 1e30, 7e4])
    plant_value(c, 0, 120, 0, [9], [-5e7])
    plant_value(c, 2, 230, 1, [5], [2e5])
    check_case(c, "V beyond f16's range")


def test_prefill_append_out_of_pool_entry_is_not_written():
    # An entry outside the pool inside the context breaks a precondition (the
    # oracle refuses it, and the two paths then read different rows); the
    # fused call must still write nothing for those tokens and nothing else.
    c = W.make_prefill_case(2, 0, [10, 40], 4, 128, 16, "bf16", seed=47, q_lens=[30, 9], name="oob")
    c.block_tables[0, 2] = c.num_blocks + 5  # positions 32..39: tokens 22..29 of the first chunk
    slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    out_f, k_f, v_f, _, k_s, v_s, _ = run_both(c)
    assert same_bytes(k_f, k_s) and same_bytes(v_f, v_s)
    k_ref = c.k_cache.copy()
    good = np.array([int(s) // 16 < c.num_blocks and int(s) >= 0 for s in slots])
    oracle.reshape_and_cache(k_ref, c.v_cache.copy(), c.new_key, c.new_value, np.where(good, slots, -1), "bf16")
    assert host(k_f, "bf16").tobytes() == k_ref.tobytes()


def test_prefill_append_refuses_shapes_without_the_matrix_kernel():
    c = W.make_prefill_case(1, 8, [4], 2, 64, 16, "f16", seed=48, name="d64")
    q = dev(c.q, "f16")
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_attention_prefill_chunk_append(torch.empty_like(q), q, dev(c.new_key, "f16"), dev(c.new_value, "f16"),
                                                dev(c.cu_q_lens), dev(c.k_cache, "f16"), dev(c.v_cache, "f16"),
                                                dev(c.block_tables), dev(c.context_lens), 8, c.max_context_len,
                                                c.scale)
    assert e.value.status == 2
