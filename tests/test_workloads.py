"""Checks of the seeded generator and the byte accounting (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

import workloads
from workloads import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_bytes_per_token_matches_printed_opt13b_example():
    g = json.load(open(os.path.join(GOLDEN, "opt13b_kv_bytes.json")))
    b = accounting.kv_bytes_per_token_model(g["hidden"], g["layers"], g["elem_bytes"])
    assert b == g["bytes_per_token"]
    assert round(b / 1024) == g["stated_per_token_kb"]
    assert round(b * g["tokens"] / 1e9, 1) == pytest.approx(g["stated_total_gb"], abs=0.1)


def test_mixed_step_composition_follows_budget_rule():
    # The golden file holds the page's worked composition of a 4,096-token
    # step (decode tokens first, then chunks capped at 1,024 tokens); the
    # generated mixed step must be exactly that step.
    g = json.load(open(os.path.join(GOLDEN, "chunked_prefill_budget.json")))
    w = workloads.make("mixed_chunked_prefill")
    assert int((w.query_lens == 1).sum()) == g["running_decodes"]
    assert w.num_tokens == g["expected_total_tokens"] <= g["budget"]
    assert list(w.query_lens[256:]) == g["expected_chunks"]
    assert max(g["expected_chunks"]) <= g["chunk_cap"]
    offsets = [p["computed"] for p in g["waiting_prompts"]]
    assert list(w.seq_lens[256:] - w.query_lens[256:]) == offsets
    lens = [p["prompt_len"] for p in g["waiting_prompts"]]
    assert all(int(L) <= P for L, P in zip(w.seq_lens[256:], lens))


@pytest.mark.parametrize("name,kw", [("tiny_decode", {}), ("llama7b_decode", {"num_seqs": 40}),
                                     ("gqa_long_decode", {"num_seqs": 8}),
                                     ("mixed_chunked_prefill", {"num_seqs": 16}),
                                     ("fp8_shared_prefix", {"num_seqs": 6})])
def test_tables_are_valid_and_disjoint(name, kw):
    w = workloads.make(name, **kw)
    B = w.block_size
    used = []
    for i in range(w.num_seqs):
        n = w.blocks_of(i)
        ids = w.block_tables[i, :n]
        assert np.all((ids >= 0) & (ids < w.num_blocks))
        assert np.all(w.block_tables[i, n:] == w.spare_block)
        used.append(ids[w.shared_prefix_len // B if w.prefix_blocks_shared else 0:])
        # waste only in the last block: fewer than B empty slots
        assert n * B - int(w.seq_lens[i]) < B
    used = np.concatenate(used)
    assert np.unique(used).size == used.size            # private blocks never collide
    assert w.spare_block not in set(used.tolist())
    if w.shared_prefix_len:
        shared = w.block_tables[:, :w.shared_prefix_len // B]
        assert np.all(shared == shared[0])
        assert not set(shared[0].tolist()) & set(used.tolist())


def test_named_shapes():
    w = workloads.make("tiny_decode")
    assert list(w.seq_lens) == [1, 7, 16, 33] and w.num_blocks == 16 and w.kv_dtype == "f32"
    w = workloads.make("llama7b_decode")
    assert w.num_seqs == 256 and w.seq_lens.min() >= 128 and w.seq_lens.max() <= 2048
    assert w.num_blocks == math.ceil(1.2 * sum(w.blocks_of(i) for i in range(256)))
    w = workloads.make("gqa_long_decode")
    assert w.num_seqs == 64 and w.seq_lens.min() >= 1024 and w.seq_lens.max() < 32768
    assert w.group == 4
    w = workloads.make("fp8_shared_prefix", block_size=64)
    assert w.shared_prefix_len == 8000 and w.kv_dtype == "fp8_e4m3" and w.k_scale == 2 ** -5
    assert np.all((w.seq_lens >= 8064) & (w.seq_lens <= 8512))


def test_values_depend_only_on_seed_and_sequence():
    a = workloads.make("fp8_shared_prefix", num_seqs=3, block_size=16, prefix=128)
    b = workloads.make("fp8_shared_prefix", num_seqs=3, block_size=64, prefix=128)
    c = workloads.make("fp8_shared_prefix", num_seqs=3, block_size=16, prefix=128,
                       placement="private")
    for i in range(3):
        for x, y in zip(a.kv_values(i), b.kv_values(i)):
            assert np.array_equal(x, y)
        for x, y in zip(a.kv_values(i), c.kv_values(i)):
            assert np.array_equal(x, y)
    assert np.array_equal(a.q_values(), b.q_values())


def test_token_writes_cover_each_slot_once():
    w = workloads.make("mixed_chunked_prefill", num_seqs=5, chunk_scale=16)
    seen = []
    new = []
    for kind, i, k, v, s in w.iter_token_writes():
        assert k.shape[0] == s.shape[0] == v.shape[0]
        seen.append(s)
        if kind == "new":
            new.append(s)
    seen = np.concatenate(seen)
    assert np.unique(seen).size == seen.size == int(w.seq_lens.sum())
    k, v, s = w.new_token_batch()
    assert np.array_equal(np.concatenate(new), s) and s.size == w.num_tokens


def test_accounting_formulas():
    w = workloads.make("mixed_chunked_prefill")
    # chunk pairs: c*o + c(c+1)/2 for the four chunks
    chunk_pairs = 524800 + 4719104 + 8913408 + 131328
    dec_pairs = int(w.seq_lens[:256].sum())
    assert accounting.workload_pairs(w) == chunk_pairs + dec_pairs
    assert accounting.workload_flops(w) == 4 * 128 * 32 * (chunk_pairs + dec_pairs)
    assert accounting.workload_kv_bytes(w) == int(w.seq_lens.sum()) * 8 * 128 * 2 * 2
    s = workloads.make("fp8_shared_prefix", num_seqs=4)
    assert accounting.workload_kv_bytes(s, unique=True) == \
        (8000 + int((s.seq_lens - 8000).sum())) * 8 * 128 * 2
    t = workloads.make("fp8_shared_prefix", num_seqs=4, placement="private")
    assert not t.prefix_blocks_shared
    assert accounting.workload_kv_bytes(t, unique=True) == accounting.workload_kv_bytes(t) == \
        int(t.seq_lens.sum()) * 8 * 128 * 2
    assert accounting.fragmentation(workloads.make("llama7b_decode")) < 0.04
