"""GPU parity of decode steps whose last partitions are cut into finer items
(the tail split), against the fp64 oracle, every row.

The split changes only how the keys of a (sequence, kv head) pair are dealt
out to work items and merged; the result is still ordinary attention over
all of the sequence's keys (itwiki "vLLM", "PagedAttention", "Block-wise
attention": the attention of a query is a sum over its blocks).  Each case
asserts that the plan did split (workspace header word 7, the split
partitions per row tile, is positive), so a change of the split rule cannot
leave these cases testing the unsplit path.
"""

import math

import numpy as np
import pytest

import oracle.cache
import workloads
from oracle import codecs
from workloads import device as wd
from workloads.generate import build

from full_oracle import assert_close, attention, fill_pools, say

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402,F401

pytestmark = pytest.mark.gpu


def split_partitions(step):
    """Split partitions per row tile the plan chose in the last call."""
    return int(step.workspace[:64].view(torch.int32)[7].item())


def run(w):
    step = wd.stage(w)
    out = step.attend()
    torch.cuda.synchronize()
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    kp, vp = fill_pools(w)
    return step, got, attention(w, kp, vp)


def log_lens(seed, n, lo, hi):
    rng = np.random.default_rng(seed)
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int64)


# Boundary lengths: around whole partitions (512, 1024, 2048 keys), around
# whole fine items (256 keys), a context shorter than one fine item, and one
# key.
EDGES = [1, 200, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097, 8191, 8192, 8193,
         9216 + 255, 9216 + 256, 9216 + 257]

CASES = [
    # kv, q, d, B, Hq, Hkv, lens, query lens (q_len * G < 65: decode rows)
    ("bf16", "bf16", 256, 16, 16, 4, "log:1024:20000:12", [1] * 10 + [3, 2]),
    ("f16", "f16", 256, 32, 8, 8, "edges", None),
    ("fp8_e4m3", "bf16", 256, 64, 8, 2, "log:9000:24000:10", [1] * 9 + [4]),
    ("bf16", "bf16", 128, 32, 32, 8, "log:9000:30000:4", [1, 2, 1, 3]),
    ("f32", "f32", 128, 16, 8, 2, "log:300:8000:10", [1] * 8 + [5, 2]),
    ("f16", "f16", 64, 16, 4, 1, "fixed:70001,3000", [1, 1]),
]


@pytest.mark.parametrize("kv,q,d,B,Hq,Hkv,lens,qlens", CASES)
def test_split_decode_every_row(kv, q, d, B, Hq, Hkv, lens, qlens):
    label = f"split kv={kv} q={q} d={d} B={B} Hq={Hq} Hkv={Hkv} lens={lens}"
    say(label)
    if lens == "edges":
        L = np.array(EDGES, dtype=np.int64)
    elif lens.startswith("fixed:"):
        L = np.array([int(x) for x in lens[6:].split(",")], dtype=np.int64)
    else:
        _, lo, hi, n = lens.split(":")
        L = log_lens(141101 + d + Hq, int(n), int(lo), int(hi))
    ql = qlens if qlens is not None else [1] * len(L)
    fp8 = kv == "fp8_e4m3"
    w = build("split", 141200 + d, L, ql, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, block_size=B,
              kv_dtype=kv, q_dtype=q, k_scale=2.0 ** -5 if fp8 else 1.0, v_scale=1.5 * 2.0 ** -5 if fp8 else 1.0)
    step, got, ref = run(w)
    S = split_partitions(step)
    say(f"  split partitions per row tile: {S}")
    assert S > 0
    assert_close(w, got, ref, label=label)


def test_full_gqa_long_decode_d256():
    # the head-dim-256 GQA step (16 q / 4 kv heads, 1k-32k contexts), where
    # the split cuts the kernel's tail, issued as the throughput measurement
    # issues it: one pa_write_and_attend call (arguments marshalled once)
    # for the new tokens' cache write and the attention, called twice
    w = workloads.make("gqa_long_decode", head_dim=256)
    say("full gqa_long_decode d256: staging", w.summary())
    step = wd.stage(w, write_new=False)
    call = step.bound_step()
    call()
    out = call()
    torch.cuda.synchronize()
    assert split_partitions(step) > 0
    nk, nv, ns = w.new_token_batch()
    blk, off = ns // w.block_size, ns % w.block_size
    assert np.array_equal(wd.to_host_bits(step.k_cache)[blk, :, off, :],
                          oracle.cache.encode_tokens(nk, w.src_dtype, w.kv_dtype, w.k_scale))
    assert np.array_equal(wd.to_host_bits(step.v_cache)[blk, :, off, :],
                          oracle.cache.encode_tokens(nv, w.src_dtype, w.kv_dtype, w.v_scale))
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    del step
    kp, vp = fill_pools(w)
    assert_close(w, got, attention(w, kp, vp), label="gqa_long_decode d256, every row")


def test_no_split_where_it_does_not_pay():
    # head dim 128 bf16 with five partitions per wave, and a step with prompt
    # chunks, keep whole partitions
    w = workloads.make("gqa_long_decode")
    step = wd.stage(w)
    step.attend()
    torch.cuda.synchronize()
    assert split_partitions(step) == 0
    w = build("split_chunks", 7, [5000, 3000, 9000], [1, 200, 1], num_q_heads=16, num_kv_heads=4, head_dim=256,
              block_size=16, kv_dtype="bf16")
    step = wd.stage(w)
    step.attend()
    torch.cuda.synchronize()
    assert split_partitions(step) == 0


def test_split_after_shared_prefix():
    # pa_attention_shared_prefix: the prefix pass's partials come first in
    # each row's list, the split suffix items after them
    P = 4096
    own = log_lens(141300, 8, 1500, 12000)
    w = build("split_pfx", 141301, P + own, [1] * 6 + [3, 2], num_q_heads=16, num_kv_heads=4, head_dim=256,
              block_size=16, kv_dtype="bf16", shared_prefix_len=P)
    step = wd.stage(w)
    step.use_shared_prefix(P)
    out = step.attend()
    torch.cuda.synchronize()
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    assert split_partitions(step) > 0
    kp, vp = fill_pools(w)
    assert_close(w, got, attention(w, kp, vp), label="split after a 4,096-token shared prefix")


@pytest.mark.parametrize("seed", range(6))
def test_random_decode_steps(seed):
    # seeded random decode-only steps around the split's conditions: head dim
    # 128 or 256, every cache type, block size 16/32/64, group 1-8, 2-24
    # sequences with contexts up to 30k and up to 4 query tokens each; every
    # row against the oracle whether or not the plan splits
    rng = np.random.default_rng([141400, seed])
    d = int(rng.choice([128, 256]))
    kv, q = [("bf16", "bf16"), ("f16", "f16"), ("fp8_e4m3", "bf16"), ("fp8_e4m3", "f16")][int(rng.integers(4))]
    B = int(rng.choice([16, 32, 64]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    n = int(rng.integers(2, 25))
    L = log_lens(141401 + seed, n, 300, 30000)
    ql = rng.integers(1, 5, size=n)
    ql = np.minimum(ql, max(1, 64 // G))           # q_len * G < 65: decode rows
    fp8 = kv == "fp8_e4m3"
    w = build("split_rand", 141402 + seed, L, ql, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d, block_size=B,
              kv_dtype=kv, q_dtype=q, k_scale=2.0 ** -5 if fp8 else 1.0, v_scale=2.0 ** -5 if fp8 else 1.0)
    step, got, ref = run(w)
    label = f"random decode seed {seed}: kv={kv} d={d} B={B} G={G} Hkv={Hkv} seqs={n}, split {split_partitions(step)}"
    say(label)
    assert_close(w, got, ref, label=label)
