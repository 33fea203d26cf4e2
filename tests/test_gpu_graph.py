"""Graph replay of the decode and prefill steps.

The library's calls only launch kernels on the caller's stream (no memset,
no allocation, no synchronisation), so a whole step can be captured once as
a HIP graph (torch.cuda.graph) and replayed. Each test captures a step,
replays it several times with eager work and synchronisations between the
replays, and checks every replay against the eager step bit for bit; the
eager step itself is checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_109_amd as pa
import workloads as W
from gpu_util import DeviceCase, check_attention, dev, device_slots, say

pytestmark = pytest.mark.gpu


def capture(step):
    """Warm the step up on a side stream, then capture it (torch's recipe)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def test_decode_step_graph_replays_match_eager():
    c = W.make_decode_case(8, 8, 128, 16, "f16", [5, 100, 700, 2048, 1, 33, 300, 1500], seed=11,
                           new_tokens=True, max_blocks_per_seq=128)
    dc = DeviceCase(c)
    seq, pos = dev(np.asarray(c.new_seq, np.int32)), dev(np.asarray(c.new_pos, np.int32))
    slots = torch.empty(c.num_seqs, dtype=torch.int64, device="cuda")
    nk, nv = dev(c.new_key, c.dtype), dev(c.new_value, c.dtype)
    ws = pa.alloc_decode_workspace(8, 8, 128, c.max_context_len, 16)
    out = torch.empty_like(dc.q)

    def step():  # translation, cache write and decode, all on the device
        pa.slot_mapping(dc.block_tables, seq, pos, c.block_size, c.num_blocks, out=slots)
        pa.reshape_and_cache(nk, nv, dc.k_cache, dc.v_cache, slots)
        pa.paged_attention_decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                                  c.max_context_len, c.scale, workspace=ws)

    say("  decode step: eager")
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    oracle.reshape_and_cache(c.k_cache, c.v_cache, c.new_key, c.new_value,
                             oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size), c.dtype)
    check_attention(eager, oracle.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale,
                                         c.dtype), c.dtype, "eager decode step")
    g = capture(step)
    other = torch.empty_like(out)
    for r in range(4):
        # Eager work between replays: clobber the output and the workspace
        # with a differently split decode.
        out.fill_(float("nan"))
        pa.paged_attention_decode(other, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                                  c.max_context_len, c.scale, workspace=ws, split_workers=7)
        torch.cuda.synchronize()
        say(f"  decode step: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"


def test_prefill_step_graph_replays_match_eager():
    c = W.make_prefill_case(3, 0, [0, 500, 1300], 4, 128, 16, "bf16", seed=5, q_lens=[100, 256, 37])
    dc = DeviceCase(c)
    slots = device_slots(c)
    nk, nv = dev(c.new_key, c.dtype), dev(c.new_value, c.dtype)
    cu = dev(c.cu_q_lens)
    max_q = int(np.diff(c.cu_q_lens).max())
    out = torch.empty_like(dc.q)

    def step():
        pa.reshape_and_cache(nk, nv, dc.k_cache, dc.v_cache, slots)
        pa.paged_attention_prefill_chunk(out, dc.q, cu, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                                         max_q, c.max_context_len, c.scale)

    say("  prefill step: eager")
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    oracle.reshape_and_cache(c.k_cache, c.v_cache, c.new_key, c.new_value,
                             oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size), c.dtype)
    check_attention(eager, oracle.prefill_chunk(c.q, c.cu_q_lens, c.k_cache, c.v_cache, c.block_tables,
                                                c.context_lens, c.scale, c.dtype), c.dtype, "eager prefill step")
    g = capture(step)
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"  prefill step: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"


def test_decode_append_step_graph_replays_match_eager():
    c = W.make_decode_case(6, 8, 128, 16, "bf16", [1, 17, 640, 2048, 33, 250], seed=13, new_tokens=True,
                           max_blocks_per_seq=128)
    dc = DeviceCase(c)
    nk, nv = dev(c.new_key, c.dtype), dev(c.new_value, c.dtype)
    slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    ws = pa.alloc_decode_workspace(6, 8, 128, c.max_context_len, 16)
    out = torch.empty_like(dc.q)

    def step():
        pa.paged_attention_decode_append(out, dc.q, nk, nv, dc.k_cache, dc.v_cache, dc.block_tables,
                                         dc.context_lens, c.max_context_len, c.scale, workspace=ws)

    say("  append step: eager")
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    oracle.reshape_and_cache(c.k_cache, c.v_cache, c.new_key, c.new_value, slots, c.dtype)
    check_attention(eager, oracle.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale,
                                         c.dtype), c.dtype, "eager append step")
    blk = torch.from_numpy(slots // 16).cuda()
    off = torch.from_numpy(slots % 16).cuda()
    g = capture(step)
    for r in range(4):
        # Eager work between replays: clobber the output and the rows the
        # step writes (it never reads them), then run another decode.
        out.fill_(float("nan"))
        dc.k_cache[blk, :, off] = float("nan")
        dc.v_cache[blk, :, off] = float("nan")
        pa.paged_attention_decode(torch.empty_like(out), dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                                  dc.context_lens, c.max_context_len, c.scale, workspace=ws, split_workers=5)
        torch.cuda.synchronize()
        say(f"  append step: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        assert torch.equal(dc.k_cache[blk, :, off].view(torch.int16), nk.view(torch.int16))
        assert torch.equal(dc.v_cache[blk, :, off].view(torch.int16), nv.view(torch.int16))


def test_prefill_append_step_graph_replays_match_eager():
    c = W.make_prefill_case(3, 0, [0, 500, 1300], 4, 128, 16, "bf16", seed=6, q_lens=[100, 256, 37])
    dc = DeviceCase(c)
    nk, nv = dev(c.new_key, c.dtype), dev(c.new_value, c.dtype)
    cu = dev(c.cu_q_lens)
    max_q = int(np.diff(c.cu_q_lens).max())
    slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    out = torch.empty_like(dc.q)

    def step():
        pa.paged_attention_prefill_chunk_append(out, dc.q, nk, nv, cu, dc.k_cache, dc.v_cache, dc.block_tables,
                                                dc.context_lens, max_q, c.max_context_len, c.scale)

    say("  prefill append step: eager")
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    oracle.reshape_and_cache(c.k_cache, c.v_cache, c.new_key, c.new_value, slots, c.dtype)
    check_attention(eager, oracle.prefill_chunk(c.q, c.cu_q_lens, c.k_cache, c.v_cache, c.block_tables,
                                                c.context_lens, c.scale, c.dtype), c.dtype, "eager prefill append")
    blk = torch.from_numpy(slots // 16).cuda()
    off = torch.from_numpy(slots % 16).cuda()
    g = capture(step)
    for r in range(4):
        # Clobber the output and the rows the step writes (it never reads them).
        out.fill_(float("nan"))
        dc.k_cache[blk, :, off] = float("nan")
        dc.v_cache[blk, :, off] = float("nan")
        torch.cuda.synchronize()
        say(f"  prefill append step: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        assert torch.equal(dc.k_cache[blk, :, off].view(torch.int16), nk.view(torch.int16))
        assert torch.equal(dc.v_cache[blk, :, off].view(torch.int16), nv.view(torch.int16))
