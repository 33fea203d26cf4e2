"""Pins for the CPU oracle: every check here comes from outside the oracle.

Sources of truth used: the integers of the pages' worked examples
(tests/golden/worked_examples.json), torch's scaled_dot_product_attention in
float64 on contiguous K/V (a library routine), numpy / torch dtype
conversions, closed forms of softmax, invariance under relabelling the
physical blocks, and numpy fancy indexing for the byte moves.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def f64(arr, dtype):
    return W.to_float32(arr, dtype).astype(np.float64)


def sdpa(q, k, v, scale, mask=None):
    """Library attention in float64. q [H, Lq, D], k/v [H, n, D]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, scale=scale).numpy()


def contiguous_kv(case, s):
    """K and V of sequence s as [H, n, D] float64, for identity placement."""
    blks = case.seq_blocks[s]
    n = int(case.context_lens[s])
    if n == 0:
        shape = (case.num_heads, 0, case.head_dim)
        return np.zeros(shape), np.zeros(shape)
    b0, nb = blks[0], len(blks)
    assert blks == list(range(b0, b0 + nb))
    out = []
    for cache in (case.k_cache, case.v_cache):
        seg = f64(cache[b0:b0 + nb], case.dtype)              # [nb, H, B, D]
        seg = seg.transpose(1, 0, 2, 3).reshape(case.num_heads, nb * case.block_size, case.head_dim)
        out.append(seg[:, :n, :])
    return out


def run_decode(case, **kw):
    return oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                         case.scale, case.dtype, **kw)


# --------------------------------------------------------------- dtype decoding

def test_f16_decoding_matches_numpy_for_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.to_f64(bits.view(np.float16), "f16")
    want = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_bf16_decoding_matches_torch_for_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.to_f64(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_f32_decoding_is_exact():
    x = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.to_f64(x, "f32"), x.astype(np.float64))


# --------------------------------------------------------------- worked examples

def test_worked_example_table_lookup():
    g = GOLDEN["table_lookup"]
    B = g["block_size"]
    assert g["position"] // B == g["logical_block"] and g["position"] % B == g["offset"]
    assert g["request_B_table"][g["logical_block"]] == g["physical_block"]
    assert oracle.slot(g["request_B_table"], g["position"], B) == g["flat_slot"]


def test_worked_example_growth():
    g = GOLDEN["growth"]
    for step in g["steps"]:
        assert oracle.slot(step["table_after"], step["position"], g["block_size"]) == step["flat_slot"]


def test_worked_example_prompt_then_decode():
    g = GOLDEN["prompt_then_decode"]
    for step in g["decode_steps"]:
        assert oracle.slot(step["table_after"], step["position"], g["block_size"]) == step["flat_slot"]


def test_worked_example_cow_slots():
    g = GOLDEN["copy_on_write"]
    for r in ("response_1", "response_2"):
        assert oracle.slot(g[r]["table_after"], g[r]["writes_position"], g["block_size"]) == g[r]["flat_slot"]


@pytest.mark.parametrize("dtype", W.DTYPES)
def test_worked_example_attention_reads_only_valid_slots(dtype):
    """Request B at context 9 reads P3 x4, P0 x4, P5 x1; everything else is
    NaN-poisoned and must not change the result."""
    g = GOLDEN["attention_reads"]
    B, N, H, D = g["block_size"], g["pool_blocks"], 2, 16
    rng = np.random.default_rng(7)
    k = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), dtype)
    v = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), dtype)
    q = W.cast(rng.standard_normal((1, H, D), dtype=np.float32), dtype)
    reads = g["reads_in_logical_order"]
    want_k = np.stack([f64(k[b, :, o, :], dtype) for b, o in reads], axis=1)  # [H, 9, D]
    want_v = np.stack([f64(v[b, :, o, :], dtype) for b, o in reads], axis=1)
    for arr in (k, v):
        for b in g["excluded_blocks"]:
            W.poison(arr, dtype, (b,))
        for o in g["excluded_slots_of_block_5"]:
            W.poison(arr, dtype, (5, slice(None), o))
    table = np.array([g["request_B_table"] + [-1]], dtype=np.int32)
    out = oracle.decode(q, k, v, table, np.array([g["context_len"]], np.int32), D ** -0.5, dtype)
    assert np.all(np.isfinite(out))
    want = sdpa(f64(q, dtype)[0][:, None, :], want_k, want_v, D ** -0.5)[:, 0, :]
    np.testing.assert_allclose(out[0], want, rtol=1e-12, atol=1e-13)


def test_block_counts_and_kv_bytes():
    for c in GOLDEN["block_counts"]["cases"]:
        assert W.blocks_needed(c["tokens"], c["block_size"]) == c["blocks"]
    g = GOLDEN["kv_bytes"]
    assert g["num_heads"] * g["head_dim"] == g["hidden"]
    per_tok = W.kv_bytes_per_token(g["num_heads"], g["head_dim"], g["bytes_per_element"], g["layers"])
    assert per_tok == g["bytes_per_token"]
    assert per_tok * g["max_tokens"] == g["bytes_per_request_at_max"]
    assert round(per_tok / 1024) == 800 and round(per_tok * g["max_tokens"] / 1e9, 1) in (1.6, 1.7)


# --------------------------------------------------------------- library attention

@pytest.mark.parametrize("dtype", W.DTYPES)
@pytest.mark.parametrize("D,B", [(64, 16), (128, 16), (128, 4), (64, 32)])
def test_decode_matches_library_attention_on_contiguous_blocks(dtype, D, B):
    lens = [1, B, B + 1, 3 * B - 1, 70]
    case = W.make_decode_case(len(lens), 3, D, B, dtype, lens, seed=11, placement="identity")
    out = run_decode(case)
    for s in range(case.num_seqs):
        K, V = contiguous_kv(case, s)
        want = sdpa(f64(case.q[s], dtype)[:, None, :], K, V, case.scale)[:, 0, :]
        np.testing.assert_allclose(out[s], want, rtol=1e-11, atol=1e-12)


def test_prefill_matches_library_causal_attention():
    H, D, B = 2, 64, 4
    for dtype in ("f16", "bf16"):
        case = W.make_prefill_case(3, 5, [3, 0, 9], H, D, B, dtype, seed=3, placement="identity",
                                   q_lens=[5, 4, 1])
        out = oracle.prefill_chunk(case.q, case.cu_q_lens, case.k_cache, case.v_cache,
                                   case.block_tables, case.context_lens, case.scale, dtype)
        for s in range(case.num_seqs):
            K, V = contiguous_kv(case, s)
            lo, hi = case.cu_q_lens[s], case.cu_q_lens[s + 1]
            ql, n = hi - lo, int(case.context_lens[s])
            c = n - ql
            mask = np.arange(n)[None, :] <= (c + np.arange(ql))[:, None]
            qs = f64(case.q[lo:hi], dtype).transpose(1, 0, 2)           # [H, ql, D]
            want = sdpa(qs, K, V, case.scale, mask).transpose(1, 0, 2)
            np.testing.assert_allclose(out[lo:hi], want, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------- invariants

@pytest.mark.parametrize("dtype", W.DTYPES)
def test_permuting_physical_blocks_is_bit_identical(dtype):
    case = W.make_decode_case(5, 4, 64, 8, dtype, [1, 8, 9, 40, 77], seed=5, extra_blocks=6)
    base = run_decode(case)
    rng = np.random.default_rng(99)
    for _ in range(3):
        perm = rng.permutation(case.num_blocks)
        k2 = np.empty_like(case.k_cache); k2[perm] = case.k_cache
        v2 = np.empty_like(case.v_cache); v2[perm] = case.v_cache
        bt2 = case.block_tables.copy()
        for s, blks in enumerate(case.seq_blocks):
            bt2[s, :len(blks)] = perm[np.asarray(blks)]
        out = oracle.decode(case.q, k2, v2, bt2, case.context_lens, case.scale, dtype)
        assert np.array_equal(out, base)


def test_poisoned_tiny_workload_is_finite_and_unchanged():
    clean = W.tiny_f32()
    dirty = W.tiny_f32(poisoned=True)
    assert np.isnan(dirty.k_cache).any() and (dirty.block_tables == -1).any()
    assert np.array_equal(run_decode(clean), run_decode(dirty))
    assert np.all(np.isfinite(run_decode(dirty)))


# --------------------------------------------------------------- closed forms

def test_single_token_returns_its_value_exactly():
    case = W.make_decode_case(3, 4, 64, 16, "f32", [1, 1, 1], seed=2)
    out = run_decode(case)
    for s in range(3):
        b = case.seq_blocks[s][0]
        assert np.array_equal(out[s], case.v_cache[b, :, 0, :].astype(np.float64))


def test_zero_query_and_equal_keys_give_mean_of_values():
    case = W.make_decode_case(2, 2, 64, 16, "f32", [37, 50], seed=4)
    case.q[0] = 0.0
    b1 = case.seq_blocks[1]
    case.k_cache[b1] = case.k_cache[b1[0], :, :1, :]   # all keys of seq 1 equal
    out = run_decode(case)
    for s in range(2):
        n = int(case.context_lens[s])
        vs = np.concatenate([case.v_cache[b] for b in case.seq_blocks[s]], axis=1)  # [H, nb*B, D]
        mean = vs[:, :n, :].astype(np.float64).mean(axis=1)
        np.testing.assert_allclose(out[s], mean, rtol=1e-13, atol=1e-14)


def test_dominant_logit_selects_its_value():
    case = W.make_decode_case(1, 1, 64, 16, "f32", [40], seed=6)
    case.q[0, 0] = 0.0
    case.q[0, 0, 0] = 1.0
    blk = case.seq_blocks[0][1]
    case.k_cache[blk, 0, 5, :] = 0.0
    case.k_cache[blk, 0, 5, 0] = 400.0   # logit 50 above the others (scale 1/8)
    out = run_decode(case)
    np.testing.assert_allclose(out[0, 0], case.v_cache[blk, 0, 5].astype(np.float64), rtol=0, atol=1e-12)


def test_empty_context_gives_zero():
    case = W.make_decode_case(2, 2, 64, 16, "f16", [0, 5], seed=8)
    out = run_decode(case)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.all(out[1] != 0)


def test_table_entry_outside_pool_is_rejected():
    case = W.make_decode_case(1, 1, 64, 16, "f32", [20], seed=9)
    case.block_tables[0, 1] = case.num_blocks
    with pytest.raises(oracle.OracleError):
        run_decode(case)


# --------------------------------------------------------------- byte moves

def test_reshape_and_cache_matches_flat_slot_indexing():
    N, H, B, D, T = 9, 3, 4, 8, 12
    rng = np.random.default_rng(12)
    for dtype in W.DTYPES:
        k = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), dtype)
        v = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), dtype)
        key = W.cast(rng.standard_normal((T, H, D), dtype=np.float32), dtype)
        val = W.cast(rng.standard_normal((T, H, D), dtype=np.float32), dtype)
        slots = rng.permutation(N * B)[:T].astype(np.int64)
        slots[[2, 7]] = -1
        want_k, want_v = k.copy(), v.copy()
        for cache, src in ((want_k, key), (want_v, val)):
            flat = cache.transpose(0, 2, 1, 3).reshape(N * B, H, D)
            flat[slots[slots >= 0]] = src[slots >= 0]
            cache[...] = flat.reshape(N, B, H, D).transpose(0, 2, 1, 3)
        oracle.reshape_and_cache(k, v, key, val, slots, dtype)
        assert k.tobytes() == want_k.tobytes() and v.tobytes() == want_v.tobytes()


def test_reshape_and_cache_rejects_bad_slots():
    k = np.zeros((2, 1, 4, 8), np.float32); v = k.copy()
    key = np.ones((2, 1, 8), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.reshape_and_cache(k, v, key, key, [3, 3], "f32")
    with pytest.raises(oracle.OracleError):
        oracle.reshape_and_cache(k, v, key, key, [0, 8], "f32")
    assert not k.any()


def test_copy_blocks_matches_numpy_indexing():
    rng = np.random.default_rng(13)
    L, N = 3, 12
    ks = [W.cast(rng.standard_normal((N, 2, 4, 8), dtype=np.float32), "f16") for _ in range(L)]
    vs = [W.cast(rng.standard_normal((N, 2, 4, 8), dtype=np.float32), "f16") for _ in range(L)]
    pairs = np.array([[1, 5], [1, 6], [2, 7], [9, 0], [1, 11]], np.int64)
    want_k = [a.copy() for a in ks]; want_v = [a.copy() for a in vs]
    for a in want_k + want_v:
        a[pairs[:, 1]] = a[pairs[:, 0]]
    oracle.copy_blocks(ks, vs, pairs)
    for a, b in zip(ks + vs, want_k + want_v):
        assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("pairs", [[[1, 2], [3, 2]], [[1, 2], [2, 3]], [[0, 12]]])
def test_copy_blocks_rejects_ambiguous_mappings(pairs):
    ks = [np.zeros((12, 1, 4, 8), np.float32)]
    with pytest.raises(oracle.OracleError):
        oracle.copy_blocks(ks, [ks[0].copy()], np.array(pairs, np.int64))


def test_copy_on_write_walkthrough():
    """Two responses share a 6-token prefix in P0, P1 (B=4). Response 1 writes
    position 6: P1 is copied into P2 first and the write lands in P2; response
    2 then writes in place into P1. Three physical blocks end up in use."""
    g = GOLDEN["copy_on_write"]
    B, H, D, N, dtype = g["block_size"], 2, 8, 6, "f16"
    rng = np.random.default_rng(21)
    k = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), dtype)
    v = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), dtype)
    pk = W.cast(rng.standard_normal((6, H, D), dtype=np.float32), dtype)
    pv = W.cast(rng.standard_normal((6, H, D), dtype=np.float32), dtype)
    a0 = W.cast(rng.standard_normal((1, H, D), dtype=np.float32), dtype)
    b0 = W.cast(rng.standard_normal((1, H, D), dtype=np.float32), dtype)
    shared = g["shared_table"]
    prefix_slots = [oracle.slot(shared, p, B) for p in range(g["prefix_tokens"])]
    oracle.reshape_and_cache(k, v, pk, pv, prefix_slots, dtype)
    p0_before = k[0].copy()
    oracle.copy_blocks([k], [v], np.array([g["response_1"]["copy"]], np.int64))
    r1, r2 = g["response_1"], g["response_2"]
    oracle.reshape_and_cache(k, v, a0, a0, [oracle.slot(r1["table_after"], r1["writes_position"], B)], dtype)
    oracle.reshape_and_cache(k, v, b0, b0, [oracle.slot(r2["table_after"], r2["writes_position"], B)], dtype)
    assert k[2, :, :2].tobytes() == k[1, :, :2].tobytes() == pk[4:6].transpose(1, 0, 2).tobytes()
    assert k[2, :, 2].tobytes() == a0[0].tobytes() and k[1, :, 2].tobytes() == b0[0].tobytes()
    assert k[0].tobytes() == p0_before.tobytes()
    used = {b for t in (r1["table_after"], r2["table_after"]) for b in t}
    assert len(used) == g["physical_blocks_in_use_after"]
    # each response attends over its own 7 tokens
    q = W.cast(rng.standard_normal((2, H, D), dtype=np.float32), dtype)
    tables = np.array([r1["table_after"], r2["table_after"]], np.int32)
    out = oracle.decode(q, k, v, tables, np.array([7, 7], np.int32), D ** -0.5, dtype)
    for s, new in enumerate((a0, b0)):
        K = np.concatenate([f64(pk, dtype), f64(new, dtype)], axis=0).transpose(1, 0, 2)
        V = np.concatenate([f64(pv, dtype), f64(new, dtype)], axis=0).transpose(1, 0, 2)
        want = sdpa(f64(q[s], dtype)[:, None, :], K, V, D ** -0.5)[:, 0, :]
        np.testing.assert_allclose(out[s], want, rtol=1e-12, atol=1e-13)


def test_swap_blocks_round_trip_restores_the_pool():
    """Swapping blocks out to a second pool and back to their own places
    leaves the first pool as it was; blocks outside the mapping never
    change, and the second pool holds exactly the swapped blocks."""
    rng = np.random.default_rng(4)
    gpu = [rng.integers(0, 255, size=(9, 2, 4, 16), dtype=np.uint8) for _ in range(2)]
    host = [np.zeros((5, 2, 4, 16), np.uint8) for _ in range(2)]
    keep = [g.copy() for g in gpu]
    out = np.array([[7, 0], [2, 3], [4, 1]])
    oracle.swap_blocks(gpu, host, out)
    for g, h in zip(gpu, host):
        assert np.array_equal(h[[0, 3, 1]], g[[7, 2, 4]]) and not h[[2, 4]].any()
    for g in gpu:
        g[[7, 2, 4]] = 0
    oracle.swap_blocks(host, gpu, out[:, ::-1])
    for g, k in zip(gpu, keep):
        assert np.array_equal(g, k)
    with pytest.raises(oracle.OracleError):
        oracle.swap_blocks(gpu, host, [[0, 1], [2, 1]])
