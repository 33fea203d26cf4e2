"""Plant plausible mistakes in a copy of the oracle's C source and check that
the pins catch every one of them.

Each mutant is compiled with gcc into a temporary directory (CPU only) and put
through a battery of pins that come from outside the oracle: the pages'
worked-example slots, numpy / torch dtype decoding, torch's float64
scaled_dot_product_attention on contiguous K/V (decode and causal prefill),
and numpy fancy indexing for the byte moves. The unmutated source must pass
the same battery.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "worked_examples.json")))
SRC = open(os.path.join(os.path.dirname(HERE), "oracle", "pa_oracle.c")).read()

MUTANTS = {
    "offset_off_by_one": ("int64_t offset_in_block = position % block_size;",
                          "int64_t offset_in_block = (position + 1) % block_size;"),
    "logical_block_off_by_one": ("int64_t logical_block = position / block_size;",
                                 "int64_t logical_block = (position + 1) / block_size;"),
    "cache_layout_transposed": (
        "return ((physical_block * num_heads + head) * block_size + offset_in_block) * head_dim;",
        "return ((physical_block * block_size + offset_in_block) * num_heads + head) * head_dim;"),
    "current_token_dropped": ("/* 1. gather each valid key through the block table and score it */\n"
                              "  for (int64_t pos = 0; pos < n; ++pos) {",
                              "/* 1. gather */\n  for (int64_t pos = 0; pos < n - 1; ++pos) {"),
    "scale_dropped": ("logits[pos] = scale * dot;", "logits[pos] = dot;"),
    "bad_normaliser": ("out[d] /= denom;", "out[d] /= (denom + 1.0);"),
    "values_from_key_cache": ("out[d] += logits[pos] * element(v_cache, v_row + d, dtype);",
                              "out[d] += logits[pos] * element(k_cache, v_row + d, dtype);"),
    "f16_exponent_bias": ("mag = ldexp((double)(1024 + frac), e - 25);",
                          "mag = ldexp((double)(1024 + frac), e - 24);"),
    "bf16_shift": ("uint32_t bits = (uint32_t)b << 16;", "uint32_t bits = (uint32_t)b << 15;"),
    "prefill_excludes_self": ("cached + j + 1, h, num_heads,", "cached + j, h, num_heads,"),
    "value_written_from_key": ("(const char *)value + (t * value_token_stride",
                               "(const char *)key + (t * key_token_stride"),
    "v_block_copied_from_k": ("(const char *)v_caches[l] + src * block_bytes",
                              "(const char *)k_caches[l] + src * block_bytes"),
    "q_row_ignored": ("dot += element(q, q_row + d, dtype)", "dot += element(q, d, dtype)"),
}


def sdpa(q, k, v, scale, mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale).numpy()


def f64(a, dtype):
    return W.to_float32(a, dtype).astype(np.float64)


def contiguous(case, cache, s):
    b0, nb, n = case.seq_blocks[s][0], len(case.seq_blocks[s]), int(case.context_lens[s])
    seg = f64(cache[b0:b0 + nb], case.dtype).transpose(1, 0, 2, 3)
    return seg.reshape(case.num_heads, nb * case.block_size, case.head_dim)[:, :n]


def battery(lib):
    """Return the list of failed pins for an oracle library."""
    failed = []

    def pin(name, ok):
        if not ok:
            failed.append(name)

    # worked-example slots
    g = GOLDEN["table_lookup"]
    pin("slot_lookup", oracle.slot(g["request_B_table"], g["position"], g["block_size"], lib=lib) == g["flat_slot"])
    for st in GOLDEN["growth"]["steps"] + GOLDEN["prompt_then_decode"]["decode_steps"]:
        pin("slot_steps", oracle.slot(st["table_after"], st["position"], 4, lib=lib) == st["flat_slot"])
    # dtype decoding
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want16 = bits.view(np.float16).astype(np.float64)
    got16 = oracle.to_f64(bits.view(np.float16), "f16", lib=lib)
    pin("f16_decode", np.array_equal(got16, want16, equal_nan=True))
    wantbf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    pin("bf16_decode", np.array_equal(oracle.to_f64(bits, "bf16", lib=lib), wantbf, equal_nan=True))
    # decode vs library attention
    for dtype, D, B in (("f32", 64, 4), ("f16", 128, 16), ("bf16", 64, 16)):
        case = W.make_decode_case(4, 2, D, B, dtype, [1, B + 1, 2 * B, 37], seed=1, placement="identity")
        try:
            out = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                case.scale, dtype, lib=lib)
        except oracle.OracleError:
            pin(f"decode_{dtype}", False)
            continue
        ok = True
        for s in range(case.num_seqs):
            want = sdpa(f64(case.q[s], dtype)[:, None], contiguous(case, case.k_cache, s),
                        contiguous(case, case.v_cache, s), case.scale)[:, 0]
            ok &= np.allclose(out[s], want, rtol=1e-10, atol=1e-12)
        pin(f"decode_{dtype}", ok)
    # causal prefill vs library attention
    case = W.make_prefill_case(2, 5, [3, 6], 2, 64, 4, "f16", seed=2, placement="identity")
    try:
        out = oracle.prefill_chunk(case.q, case.cu_q_lens, case.k_cache, case.v_cache, case.block_tables,
                                   case.context_lens, case.scale, "f16", lib=lib)
        ok = True
        for s in range(2):
            lo, hi = case.cu_q_lens[s], case.cu_q_lens[s + 1]
            n, ql = int(case.context_lens[s]), hi - lo
            mask = np.arange(n)[None, :] <= (n - ql + np.arange(ql))[:, None]
            want = sdpa(f64(case.q[lo:hi], "f16").transpose(1, 0, 2), contiguous(case, case.k_cache, s),
                        contiguous(case, case.v_cache, s), case.scale, mask).transpose(1, 0, 2)
            ok &= np.allclose(out[lo:hi], want, rtol=1e-10, atol=1e-12)
        pin("prefill", ok)
    except oracle.OracleError:
        pin("prefill", False)
    # cache write vs flat-slot indexing
    rng = np.random.default_rng(3)
    N, H, B, D, T = 6, 2, 4, 8, 7
    k = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), "f16")
    v = W.cast(rng.standard_normal((N, H, B, D), dtype=np.float32), "f16")
    key = W.cast(rng.standard_normal((T, H, D), dtype=np.float32), "f16")
    val = W.cast(rng.standard_normal((T, H, D), dtype=np.float32), "f16")
    slots = rng.permutation(N * B)[:T].astype(np.int64)
    wk, wv = k.copy(), v.copy()
    for cache, src in ((wk, key), (wv, val)):
        flat = cache.transpose(0, 2, 1, 3).reshape(N * B, H, D)
        flat[slots] = src
        cache[...] = flat.reshape(N, B, H, D).transpose(0, 2, 1, 3)
    oracle.reshape_and_cache(k, v, key, val, slots, "f16", lib=lib)
    pin("reshape", k.tobytes() == wk.tobytes() and v.tobytes() == wv.tobytes())
    # block copy vs numpy indexing
    kc = [k.copy(), k.copy() + 1]
    vc = [v.copy(), v.copy() + 2]
    pairs = np.array([[0, 3], [0, 4], [1, 5]], np.int64)
    wk = [a.copy() for a in kc]; wv = [a.copy() for a in vc]
    for a in wk + wv:
        a[pairs[:, 1]] = a[pairs[:, 0]]
    oracle.copy_blocks(kc, vc, pairs, lib=lib)
    pin("copy_blocks", all(a.tobytes() == b.tobytes() for a, b in zip(kc + vc, wk + wv)))
    return failed


def _build(tmp_path, name, src_text):
    src = tmp_path / f"{name}.c"
    src.write_text(src_text)
    return oracle.load(oracle.build(force=True, src=str(src), out=str(tmp_path / f"lib{name}.so")))


def test_unmutated_oracle_passes_the_battery(tmp_path):
    assert battery(_build(tmp_path, "clean", SRC)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor for {name} not unique in the oracle source"
    failed = battery(_build(tmp_path, name, SRC.replace(old, new)))
    assert failed, f"mutant {name} passed every pin"
