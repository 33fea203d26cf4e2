"""The allocation-free decode entry point (pa_paged_attention_decode_noalloc)
against the workspace one (pa_paged_attention_decode), through the C ABI.

Both run the same kernels at the same split, so their outputs must agree
byte for byte; both are also checked against the oracle. Two calls in a
row, the second on a smaller batch, show that the library's fixed
workspace, which keeps the previous call's contents, needs no clearing.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_109_amd as pa
import workloads as W
from gpu_util import DeviceCase, check_attention, say

pytestmark = pytest.mark.gpu


def run_both(c, split_workers=0):
    dc = DeviceCase(c)
    say(f"  noalloc vs workspace decode: S={c.num_seqs} H={c.num_heads} D={c.head_dim} B={c.block_size} "
        f"{c.dtype} max_ctx={c.max_context_len} split_workers={split_workers}")
    ref_out = torch.full_like(dc.q, float("nan"))
    pa.paged_attention_decode(ref_out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                              c.max_context_len, c.scale, split_workers=split_workers)
    out = torch.full_like(dc.q, float("nan"))
    pa.paged_attention_decode_noalloc(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                                      c.max_context_len, c.scale, split_workers=split_workers)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.element_size() == 2 else out.view(torch.int32),
                       ref_out.view(torch.int16) if out.element_size() == 2 else ref_out.view(torch.int32))
    ref = oracle.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale, c.dtype)
    say("  max err", check_attention(out, ref, c.dtype, f"noalloc {c.name}"))


@pytest.mark.parametrize("split_workers", [0, 37])
def test_noalloc_matches_workspace_decode_twice_second_smaller(split_workers):
    big = W.make_decode_case(48, 8, 128, 16, "f16", lambda r, n: r.integers(1, 1500, n), seed=21,
                             max_blocks_per_seq=96)
    run_both(big, split_workers)
    small = W.make_decode_case(5, 4, 128, 16, "f16", [1, 17, 64, 300, 0], seed=22, max_blocks_per_seq=20)
    run_both(small, split_workers)


def test_noalloc_other_shapes_and_plan_kernel():
    # bf16 at head_dim 64 with block size 32, then a batch of more than 1024
    # sequences, whose plan is written by its own kernel into the fixed array.
    run_both(W.make_decode_case(9, 3, 64, 32, "bf16", [2, 33, 64, 65, 700, 1, 128, 1000, 5], seed=23,
                                max_blocks_per_seq=40))
    run_both(W.make_decode_case(1100, 2, 128, 16, "f16", lambda r, n: r.integers(0, 60, n), seed=24,
                                max_blocks_per_seq=4))


def test_noalloc_empty_batch_is_a_no_op():
    c = W.make_decode_case(2, 2, 128, 16, "f16", [3, 4], seed=25, max_blocks_per_seq=1)
    dc = DeviceCase(c)
    before = dc.out.clone()
    pa.paged_attention_decode_noalloc(dc.out[:0], dc.q[:0], dc.k_cache, dc.v_cache, dc.block_tables[:0],
                                      dc.context_lens[:0], c.max_context_len, c.scale)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), dc.out.view(torch.int16))
