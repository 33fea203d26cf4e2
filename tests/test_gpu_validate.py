"""The debug validation (PA_DEBUG_VALIDATE=1): every entry point that reads
device index arrays checks the data-dependent preconditions before it
enqueues anything. Valid inputs give the same bytes as without the check;
each violation is refused with PA_ERR_INVALID_ARG, a message naming it, and
no write to the output. Without the variable the same call is not checked
(the kernels clip or skip such data, as the other GPU tests show)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_109_amd as pa
import workloads as W
from gpu_util import dev, say
from paged_kv_cache_109_amd import _binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("PA_DEBUG_VALIDATE", "1")


def refused(fn, text):
    with pytest.raises(pa.PagedAttnError) as e:
        fn()
    assert e.value.status == B.PA_ERR_INVALID_ARG, str(e.value)
    assert "PA_DEBUG_VALIDATE" in str(e.value) and text in str(e.value), str(e.value)
    say(f"  refused: {e.value}")


def decode_case():
    c = W.make_decode_case(4, 2, 64, 16, "f16", [40, 17, 1, 64], seed=3, extra_blocks=3, max_blocks_per_seq=5)
    return c, dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_tables), dev(c.context_lens)


def test_decode(validate):
    c, q, k, v, bt, ctx = decode_case()
    out = pa.paged_attention_decode(torch.empty_like(q), q, k, v, bt, ctx, 64, c.scale)
    torch.cuda.synchronize()
    plain = torch.empty_like(q)
    with pytest.MonkeyPatch.context() as m:
        m.delenv("PA_DEBUG_VALIDATE")
        pa.paged_attention_decode(plain, q, k, v, bt, ctx, 64, c.scale)
        torch.cuda.synchronize()
    assert torch.equal(out, plain)

    sentinel = torch.full_like(q, 7.0)
    bad = bt.clone()
    bad[1, 1] = c.k_cache.shape[0]  # position 16 of a 17-token context
    refused(lambda: pa.paged_attention_decode(sentinel, q, k, v, bad, ctx, 64, c.scale), "block_tables[1][1]")
    refused(lambda: pa.paged_attention_decode(sentinel, q, k, v, bt, ctx, 63, c.scale), "context_lens[3] = 64")
    neg = ctx.clone()
    neg[2] = -1
    refused(lambda: pa.paged_attention_decode(sentinel, q, k, v, bt, neg, 64, c.scale), "context_lens[2] = -1")
    refused(lambda: pa.paged_attention_decode(sentinel, q, k, v, bt, ctx, 81, c.scale), "exceeds max_blocks_per_seq")
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


def test_unchecked_without_the_variable(monkeypatch):
    monkeypatch.delenv("PA_DEBUG_VALIDATE", raising=False)
    c, q, k, v, bt, ctx = decode_case()
    pa.paged_attention_decode(torch.empty_like(q), q, k, v, bt, ctx, 63, c.scale)  # context 64 is clipped
    torch.cuda.synchronize()


def shared_case():
    rng = np.random.default_rng(5)
    H, D, Bs, N = 2, 64, 16, 10
    k = W.cast(rng.standard_normal((N, H, Bs, D), dtype=np.float32), "f16")
    v = W.cast(rng.standard_normal((N, H, Bs, D), dtype=np.float32), "f16")
    q = W.cast(rng.standard_normal((3, H, D), dtype=np.float32), "f16")
    tables = np.array([[5, 6, 7], [5, 6, 8], [5, 6, 9]], np.int32)
    lens = np.array([40, 35, 33], np.int32)
    gm, gp, st, maxp = pa.shared_prefix_groups(tables, lens, [[0, 1, 2]], Bs)
    assert gp.tolist() == [32]
    return dict(q=dev(q), k=dev(k), v=dev(v), bt=dev(tables), ctx=dev(lens), gm=gm, gp=gp, st=st, maxp=maxp,
                scale=1.0 / np.sqrt(D))


def run_shared(s, out, gm=None, gp=None, st=None, bt=None, maxp=None):
    gm = s["gm"] if gm is None else gm
    gp = s["gp"] if gp is None else gp
    st = s["st"] if st is None else st
    return pa.paged_attention_decode_shared(out, s["q"], s["k"], s["v"], s["bt"] if bt is None else bt, s["ctx"], 40,
                                            s["scale"], dev(np.asarray(gm, np.int32)), dev(np.asarray(gp, np.int32)),
                                            dev(np.asarray(st, np.int32)), s["maxp"] if maxp is None else maxp)


def test_decode_shared(validate):
    s = shared_case()
    out = run_shared(s, torch.empty_like(s["q"]))
    torch.cuda.synchronize()
    plain = torch.empty_like(s["q"])
    with pytest.MonkeyPatch.context() as m:
        m.delenv("PA_DEBUG_VALIDATE")
        run_shared(s, plain)
        torch.cuda.synchronize()
    assert torch.equal(out, plain)

    sentinel = torch.full_like(s["q"], 7.0)
    pad = [-1] * 5
    refused(lambda: run_shared(s, sentinel, gm=[[0, -1, 1] + pad]), "leading run")
    refused(lambda: run_shared(s, sentinel, gm=[[0, 1, -1] + pad, [1, 2, -1] + pad], gp=[32, 32]), "more than one group")
    refused(lambda: run_shared(s, sentinel, gp=[24], st=[24, 24, 24]), "not a multiple of 16")
    refused(lambda: run_shared(s, sentinel, gp=[48], st=[48, 48, 48], maxp=48), "exceeds context_lens[0] = 40")
    refused(lambda: run_shared(s, sentinel, st=[32, 32, 0]), "seq_starts[2]")
    bt = s["bt"].clone()
    bt[2, 1] = 4
    refused(lambda: run_shared(s, sentinel, bt=bt), "differ at table entry 1")
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


def test_reshape_and_cache(validate):
    k = torch.zeros(4, 2, 16, 64, dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    key = torch.ones(3, 2, 64, dtype=torch.float16, device="cuda")
    pa.reshape_and_cache(key, key, k, v, torch.tensor([5, -1, 63], dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert int((k != 0).sum()) == 2 * 2 * 64
    k.zero_()
    refused(lambda: pa.reshape_and_cache(key, key, k, v, torch.tensor([5, 9, 5], dtype=torch.int64, device="cuda")),
            "slot 5 appears twice")
    refused(lambda: pa.reshape_and_cache(key, key, k, v, torch.tensor([5, 64, 1], dtype=torch.int64, device="cuda")),
            "slot_mapping[1] = 64 outside the pool")
    torch.cuda.synchronize()
    assert int((k != 0).sum()) == 0


def test_copy_blocks(validate):
    k = torch.arange(24 * 16, dtype=torch.float32, device="cuda").reshape(24, 1, 16, 1).repeat(1, 1, 1, 4)
    v = k.clone()
    before = k.clone()
    pa.copy_blocks([k], [v], torch.tensor([[2, 9], [2, 10]], dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(k[9], before[2]) and torch.equal(k[10], before[2])
    k.copy_(before)
    for pairs, text in (([[2, 9], [3, 9]], "destination block 9 appears twice"),
                        ([[2, 9], [9, 4]], "block 9 is both a source and a destination"),
                        ([[2, 24]], "outside [0, 24)")):
        refused(lambda: pa.copy_blocks([k], [v], torch.tensor(pairs, dtype=torch.int64, device="cuda")), text)
    torch.cuda.synchronize()
    assert torch.equal(k, before)


def test_swap_blocks(validate):
    src = torch.arange(6 * 16 * 8, dtype=torch.float16, device="cuda").reshape(6, 1, 16, 8)
    host = torch.zeros((4, 1, 16, 8), dtype=torch.float16, pin_memory=True)
    pa.swap_blocks([src], [host], torch.tensor([[5, 0], [1, 3]], dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(host[0], src[5].cpu()) and torch.equal(host[3], src[1].cpu())
    host.zero_()
    refused(lambda: pa.swap_blocks([src], [host], torch.tensor([[5, 0], [1, 0]], dtype=torch.int64, device="cuda")),
            "destination block 0 appears twice")
    refused(lambda: pa.swap_blocks([src], [host], torch.tensor([[6, 0]], dtype=torch.int64, device="cuda")),
            "source block 6 outside [0, 6)")
    refused(lambda: pa.swap_blocks([src], [host], torch.tensor([[1, 4]], dtype=torch.int64, device="cuda")),
            "destination block 4 outside [0, 4)")
    torch.cuda.synchronize()
    assert int((host != 0).sum()) == 0


def test_prefill_chunk(validate):
    c = W.make_prefill_case(2, 0, [30, 5], 2, 128, 16, "bf16", seed=4, q_lens=[10, 7], name="validate")
    q, k, v = dev(c.q, "bf16"), dev(c.k_cache, "bf16"), dev(c.v_cache, "bf16")
    cu, bt, ctx = dev(c.cu_q_lens), dev(c.block_tables), dev(c.context_lens)
    max_ctx = int(c.context_lens.max())

    def call(out, cu=cu, bt=bt, ctx=ctx):
        return pa.paged_attention_prefill_chunk(out, q, cu, k, v, bt, ctx, 10, max_ctx, c.scale)

    out = call(torch.empty_like(q))
    torch.cuda.synchronize()
    plain = torch.empty_like(q)
    with pytest.MonkeyPatch.context() as m:
        m.delenv("PA_DEBUG_VALIDATE")
        call(plain)
        torch.cuda.synchronize()
    assert torch.equal(out, plain)

    sentinel = torch.full_like(q, 7.0)
    refused(lambda: call(sentinel, cu=torch.tensor([0, 10, 16], dtype=torch.int32, device="cuda")),
            "cu_q_lens must run from 0 to total_q = 17")
    short = ctx.clone()
    short[1] = 5
    refused(lambda: call(sentinel, ctx=short), "q_len 7 exceeds context_lens = 5")
    bad = bt.clone()
    bad[0, 2] = c.k_cache.shape[0]
    refused(lambda: call(sentinel, bt=bad), "block_tables[0][2]")
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


def test_decode_append(validate):
    c, q, k, v, bt, ctx = decode_case()
    rng = np.random.default_rng(9)
    nk = dev(W.normal_cast(rng, (4, 2, 64), "f16"))
    nv = dev(W.normal_cast(rng, (4, 2, 64), "f16"))
    k2, v2 = k.clone(), v.clone()
    out = pa.paged_attention_decode_append(torch.empty_like(q), q, nk, nv, k2, v2, bt, ctx, 64, c.scale)
    torch.cuda.synchronize()
    plain, k3, v3 = torch.empty_like(q), k.clone(), v.clone()
    with pytest.MonkeyPatch.context() as m:
        m.delenv("PA_DEBUG_VALIDATE")
        pa.paged_attention_decode_append(plain, q, nk, nv, k3, v3, bt, ctx, 64, c.scale)
        torch.cuda.synchronize()
    assert torch.equal(out, plain) and torch.equal(k2, k3) and torch.equal(v2, v3)

    # A refused call writes neither the output nor the caches.
    sentinel, k4, v4 = torch.full_like(q, 7.0), k.clone(), v.clone()
    bad = bt.clone()
    bad[1, 1] = c.k_cache.shape[0]  # position 16 of a 17-token context: the newest token's block
    refused(lambda: pa.paged_attention_decode_append(sentinel, q, nk, nv, k4, v4, bad, ctx, 64, c.scale),
            "block_tables[1][1]")
    refused(lambda: pa.paged_attention_decode_append(sentinel, q, nk, nv, k4, v4, bt, ctx, 63, c.scale),
            "context_lens[3] = 64")
    # Copy-on-write forgotten: sequence 0 also reads the block that receives
    # sequence 1's newest token (position 16, its second block).
    shared = bt.clone()
    shared[0, 1] = bt[1, 1]
    refused(lambda: pa.paged_attention_decode_append(sentinel, q, nk, nv, k4, v4, shared, ctx, 64, c.scale),
            "sequence 1 writes position 16 into block")
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all()) and torch.equal(k4, k) and torch.equal(v4, v)


def test_prefill_chunk_append(validate):
    c = W.make_prefill_case(2, 0, [30, 5], 2, 128, 16, "bf16", seed=4, q_lens=[10, 7], name="validate_append")
    q, k, v = dev(c.q, "bf16"), dev(c.k_cache, "bf16"), dev(c.v_cache, "bf16")
    nk, nv = dev(c.new_key, "bf16"), dev(c.new_value, "bf16")
    cu, bt, ctx = dev(c.cu_q_lens), dev(c.block_tables), dev(c.context_lens)
    max_ctx = int(c.context_lens.max())

    def call(out, kc, vc, bt=bt):
        return pa.paged_attention_prefill_chunk_append(out, q, nk, nv, cu, kc, vc, bt, ctx, 10, max_ctx, c.scale)

    k1, v1 = k.clone(), v.clone()
    out = call(torch.empty_like(q), k1, v1)
    torch.cuda.synchronize()
    k2, v2, plain = k.clone(), v.clone(), torch.empty_like(q)
    with pytest.MonkeyPatch.context() as m:
        m.delenv("PA_DEBUG_VALIDATE")
        call(plain, k2, v2)
        torch.cuda.synchronize()
    assert torch.equal(out, plain) and torch.equal(k1, k2) and torch.equal(v1, v2)

    sentinel, k3, v3 = torch.full_like(q, 7.0), k.clone(), v.clone()
    bad = bt.clone()
    bad[0, 2] = c.k_cache.shape[0]
    refused(lambda: call(sentinel, k3, v3, bt=bad), "block_tables[0][2]")
    # Sequence 1 reads the block that receives sequence 0's chunk positions
    # 30 and 31.
    shared = bt.clone()
    shared[1, 0] = bt[0, 1]
    refused(lambda: call(sentinel, k3, v3, bt=shared), "sequence 0 writes position 30 into block")
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all()) and torch.equal(k3, k) and torch.equal(v3, v)

    # One sequence whose table names one block twice inside its chunk writes
    # a slot twice.
    c1 = W.make_prefill_case(1, 0, [0], 2, 128, 16, "bf16", seed=5, q_lens=[20], name="twice")
    q1, k1, v1 = dev(c1.q, "bf16"), dev(c1.k_cache, "bf16"), dev(c1.v_cache, "bf16")
    twice = dev(c1.block_tables)
    twice[0, 1] = twice[0, 0]
    sentinel1, kk, vv = torch.full_like(q1, 7.0), k1.clone(), v1.clone()
    refused(lambda: pa.paged_attention_prefill_chunk_append(
        sentinel1, q1, dev(c1.new_key, "bf16"), dev(c1.new_value, "bf16"), dev(c1.cu_q_lens), kk, vv, twice,
        dev(c1.context_lens), 20, 20, c1.scale), "is written twice (sequence 0, position 16)")
    torch.cuda.synchronize()
    assert bool((sentinel1 == 7.0).all()) and torch.equal(kk, k1) and torch.equal(vv, v1)
