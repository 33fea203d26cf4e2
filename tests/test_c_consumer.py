"""libpagedattn from plain C: include/pagedattn.h compiled as C11 with gcc
-Wall -Werror, the library linked directly, no Python or torch in the
process (tests/c_consumer/decode_step.c).

The CPU test compiles the consumer itself and runs its host-side checks.
The GPU test runs the binary that build() made: one decode step (the slots
of one new token per sequence, their cache write, then the decode) from raw
files, whose slots and written caches must equal the oracle's bit for bit
and whose output must match the oracle's decode.
"""
import importlib.util
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def _builder():
    spec = importlib.util.spec_from_file_location("_c_consumer_build", os.path.join(HERE, "c_consumer", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_header_compiles_as_c_and_host_checks_pass(tmp_path):
    exe = _builder().build(str(tmp_path / "decode_step"))
    r = subprocess.run([exe, "check"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "check ok" in r.stdout


@pytest.mark.gpu
def test_decode_step_from_c_matches_the_oracle(tmp_path):
    from gpu_util import say
    exe = _builder().BIN
    assert os.path.exists(exe), "tests/c_consumer/decode_step is missing: run __graft_entry__.build()"
    c = W.make_decode_case(5, 4, 128, 16, "f16", [1, 17, 300, 1000, 48], seed=21, new_tokens=True,
                           extra_blocks=3, max_blocks_per_seq=64)
    slots = oracle.slots(c.block_tables, c.new_seq, c.new_pos, c.block_size)
    d = tmp_path
    (d / "meta.txt").write_text(f"{c.num_seqs} {c.num_heads} {c.head_dim} {c.block_size} {c.num_blocks} "
                                f"{c.max_blocks_per_seq} {c.max_context_len} {c.scale!r}\n")
    for name, arr in (("q", c.q), ("k", c.k_cache), ("v", c.v_cache), ("tables", c.block_tables.astype(np.int32)),
                      ("ctx", c.context_lens.astype(np.int32)), ("new_k", c.new_key), ("new_v", c.new_value),
                      ("seq", c.new_seq.astype(np.int32)), ("pos", c.new_pos.astype(np.int32))):
        np.ascontiguousarray(arr).tofile(d / f"{name}.bin")
    say(f"  C consumer: {exe} run {d}")
    r = subprocess.run([exe, "run", str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert np.array_equal(np.fromfile(d / "slots.bin", np.int64), slots)
    k_ref, v_ref = c.k_cache.copy(), c.v_cache.copy()
    oracle.reshape_and_cache(k_ref, v_ref, c.new_key, c.new_value, slots, "f16")
    assert np.fromfile(d / "k_out.bin", np.uint8).tobytes() == k_ref.tobytes()
    assert np.fromfile(d / "v_out.bin", np.uint8).tobytes() == v_ref.tobytes()
    out = np.fromfile(d / "out.bin", np.float16).reshape(c.q.shape).astype(np.float64)
    ref = oracle.decode(c.q, k_ref, v_ref, c.block_tables, c.context_lens, c.scale, "f16")
    ref16 = ref.astype(np.float16).astype(np.float64)
    err = np.abs(out - ref16)
    ok = (err <= 2e-3) | (err <= 1e-2 * np.abs(ref16))
    assert ok.all(), f"{int((~ok).sum())} elements out of tolerance, max abs {err.max():.3g}"
    say(f"  C consumer: caches bit-exact, output max abs {err.max():.2e}")
