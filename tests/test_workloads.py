"""The seeded generators: determinism, shapes, ranges, placement validity and
the bf16 cast, checked against torch's own float32 -> bfloat16 rounding."""
import numpy as np
import torch

import workloads as W


def test_bf16_cast_matches_torch_rounding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    # exact ties: low 16 bits 0x8000 with even and odd upper halves
    ties = (np.arange(64, dtype=np.uint32) << np.uint32(16) | np.uint32(0x3F808000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), want)
    assert np.array_equal(W.to_float32(want, "bf16"), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def _check_tables(case):
    seen = set()
    for s, blks in enumerate(case.seq_blocks):
        n = int(case.context_lens[s])
        assert len(blks) == W.blocks_needed(n, case.block_size)
        assert list(case.block_tables[s, :len(blks)]) == blks
        assert all(0 <= b < case.num_blocks for b in blks)
        assert not (set(blks) & seen)
        seen |= set(blks)


def test_tiny_workload():
    c = W.tiny_f32()
    assert c.q.shape == (4, 8, 64) and c.k_cache.shape == (64, 8, 16, 64) and c.q.dtype == np.float32
    assert c.context_lens.min() >= 1 and c.context_lens.max() <= 100
    _check_tables(c)
    again = W.tiny_f32()
    assert np.array_equal(c.k_cache, again.k_cache) and np.array_equal(c.block_tables, again.block_tables)


def test_poison_marks_exactly_the_unused_slots():
    c = W.tiny_f32(poisoned=True)
    mask = W.valid_slot_mask(c)
    nan = np.isnan(c.k_cache).all(axis=(1, 3))  # [N, B]
    assert np.array_equal(nan, ~mask)
    assert (c.block_tables == -1).sum() == c.block_tables.size - sum(len(b) for b in c.seq_blocks)


def test_opt13b_workload_shapes():
    c = W.make_decode_case(64, 40, 128, 16, "f16", lambda r, n: r.integers(1, 2049, size=n),
                           seed=0, max_blocks_per_seq=128, new_tokens=True, pool_blocks=None)
    assert c.num_blocks == sum(W.blocks_needed(n, 16) for n in c.context_lens)
    _check_tables(c)
    assert c.new_key.shape == (64, 40, 128) and np.array_equal(c.new_pos, c.context_lens - 1)


def test_parallel_sampling_structure():
    c = W.parallel_sampling(groups=3, samples=6, num_heads=2, head_dim=64, prompt_len=512)
    assert c.num_seqs == 18 and c.block_mapping.shape == (15, 2)
    for g in range(3):
        rows = c.block_tables[g * 6:(g + 1) * 6]
        assert (rows[:, :31] == rows[0, :31]).all()       # shared prompt blocks
        assert len(set(rows[:, 31])) == 6                 # own last prompt block
        srcs = c.block_mapping[g * 5:(g + 1) * 5, 0]
        assert (srcs == rows[0, 31]).all() and list(c.block_mapping[g * 5:(g + 1) * 5, 1]) == list(rows[1:, 31])
    dst = c.block_mapping[:, 1]
    assert len(set(dst)) == len(dst) and not set(dst) & set(c.block_mapping[:, 0])


def test_prefill_case_structure():
    c = W.make_prefill_case(3, 8, [0, 5, 17], 2, 64, 16, "bf16", seed=1)
    assert list(c.cu_q_lens) == [0, 8, 16, 24] and list(c.context_lens) == [8, 13, 25]
    assert list(c.new_pos[:8]) == list(range(8)) and list(c.new_pos[8:16]) == list(range(5, 13))
