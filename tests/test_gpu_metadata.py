"""GPU parity of the step-input builders against the oracle (bit-exact).

pa_apply_block_table_writes from device and from page-locked host staging,
pa_prepare_step on scheduler-like states (including more than 1,024 requests
and tokens past the scheduled total), and the built inputs driving the cache
write and attention of a step end to end.
"""

import sys

import numpy as np
import pytest

import oracle
from oracle import codecs
from oracle import metadata as M
from workloads import device as wd
from workloads.generate import random_mixed

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def i32(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


@pytest.mark.parametrize("where", ["device", "pinned"])
def test_staged_writes_bit_exact(where):
    rng = np.random.default_rng(11)
    R, W = 300, 96
    table = rng.integers(0, 1 << 20, size=(R, W)).astype(np.int32)
    n = 500
    rows = rng.integers(-2, R + 2, size=n)             # a few rows outside the table
    lens = rng.integers(0, 6, size=n)
    starts = rng.integers(-1, W, size=n)               # some start before 0 or run past the width
    # runs may not overlap (the GPU leaves either value where they do): one run per row
    keep = np.unique(rows, return_index=True)[1]
    rows, lens, starts = rows[keep], lens[keep], starts[keep]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    vals = rng.integers(0, 1 << 20, size=int(offs[-1])).astype(np.int32)
    ref = M.apply_block_table_writes(table, rows, starts, offs, vals)
    g = i32(table)
    dev = "cpu" if where == "pinned" else "cuda"
    staged = [i32(x, dev) for x in (rows, starts, offs, vals)]
    if where == "pinned":
        staged = [t.pin_memory() for t in staged]
    say("staged writes from", where, "runs", len(rows), "values", len(vals))
    pa.apply_block_table_writes(g, *staged)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), ref)


@pytest.mark.parametrize("R,W,live,extra", [(64, 32, 40, 0), (2048, 128, 1500, 0), (16, 8, 9, 5)])
def test_prepare_step_bit_exact(R, W, live, extra):
    rng = np.random.default_rng(R)
    table = rng.integers(0, 1 << 22, size=(R, W)).astype(np.int32)
    idx = rng.permutation(R)[:live].astype(np.int32)
    done = rng.integers(0, W * 16 - 80, size=R).astype(np.int32)
    sched = np.where(rng.random(live) < 0.8, 1, rng.integers(1, 80, size=live)).astype(np.int32)
    if extra:
        done[idx[0]] = W * 16 - 3                     # runs past the table's width
    T = int(sched.sum()) + extra                     # tokens past the scheduled total
    ref = M.prepare_step(table, idx, done, sched, T, 16)
    say("prepare_step", R, W, live, T)
    got = pa.prepare_step(i32(table), i32(idx), i32(done), i32(sched), T, 16)
    torch.cuda.synchronize()
    for name, r, g in zip(("qsl", "seq_lens", "positions", "slot_mapping", "tables"), ref, got):
        assert np.array_equal(g.cpu().numpy(), r), name


def test_built_inputs_drive_a_step_end_to_end():
    """A mixed step whose seq_lens, query_start_loc, block tables and slot
    mapping come from pa_prepare_step (persistent slots scattered over a
    larger table): cache write byte-exact, attention within 1e-2 of the oracle."""
    w = random_mixed(21, num_decode=9, chunk_specs=[(0, 24), (70, 40)], max_decode_len=500, num_q_heads=16,
                     num_kv_heads=4, head_dim=128, block_size=16, kv_dtype="bf16")
    R = w.num_seqs + 5
    perm = np.random.default_rng(1).permutation(R)[:w.num_seqs].astype(np.int32)
    table = np.zeros((R, w.block_tables.shape[1]), np.int32)
    table[perm] = w.block_tables
    done = np.zeros(R, np.int32)
    done[perm] = w.seq_lens - w.query_lens
    qsl, lens, pos, slots, tables = pa.prepare_step(i32(table), i32(perm), i32(done), i32(w.query_lens),
                                                    w.num_tokens, w.block_size)
    step = wd.stage(w, write_new=False)
    nk, nv, _ = w.new_token_batch()
    pa.reshape_and_cache(wd.to_device(nk, w.src_dtype, "cuda"), wd.to_device(nv, w.src_dtype, "cuda"),
                         step.k_cache, step.v_cache, slots)
    out = pa.attention(wd.to_device(w.q_values(), w.q_dtype, "cuda"), step.k_cache, step.v_cache, tables, lens,
                       qsl, w.scale, max_seq_len=w.max_seq_len, max_query_len=w.max_query_len)
    torch.cuda.synchronize()
    kp, vp = oracle.cache.fill_pools(w)
    assert np.array_equal(wd.to_host_bits(step.k_cache), kp) and np.array_equal(wd.to_host_bits(step.v_cache), vp)
    ref = oracle.attention.paged_attention(w.q_values(), w.q_dtype, kp, vp, w.kv_dtype, w.block_tables, w.seq_lens,
                                           w.query_start_loc, w.block_size, w.scale)
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    err = np.abs(got - ref).max()
    say(f"step from built inputs: max-abs err {err:.3e}")
    assert not np.isnan(got).any() and err <= 1e-2
