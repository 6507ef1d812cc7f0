"""GPU parity on seeded random steps: shapes, dtypes, block sizes and length
mixes drawn at random, each step checked against the fp64 oracle.

Every draw is a valid input the library supports: head dim 64/128/256, block
size 16/32/64, 1-8 query heads per kv head, KV in fp32 (head dim <= 128),
fp16, bf16 or fp8-e4m3 with a scale, and per sequence one of: no query
tokens, one decode token, a short multi-token run, or a prompt chunk, over
contexts from 1 to about 20,000 keys.  The tolerance is the fixed one of the
KV dtype (2e-3 fp32/fp16, 1e-2 bf16, 4e-2 fp8).
"""

import sys

import numpy as np
import pytest

import oracle
from oracle import codecs
from workloads import device as wd
from workloads.generate import build

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402,F401

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-3, "f16": 2e-3, "bf16": 1e-2, "fp8_e4m3": 4e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def draw_step(seed):
    rng = np.random.default_rng([seed, 7])
    d = int(rng.choice([64, 128, 256]))
    B = int(rng.choice([16, 32, 64]))
    kvs = ["f16", "bf16", "fp8_e4m3"] + (["f32"] if d <= 128 else [])
    kv = str(rng.choice(kvs))
    q = {"f32": "f32", "f16": "f16", "bf16": "bf16"}.get(kv) or str(rng.choice(["bf16", "f16"]))
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    n = int(rng.integers(1, 25))
    lens, qlens = [], []
    for _ in range(n):
        kind = rng.choice(["none", "decode", "spec", "chunk"], p=[0.05, 0.55, 0.15, 0.25])
        ql = {"none": 0, "decode": 1, "spec": int(rng.integers(2, 9)), "chunk": int(rng.integers(16, 301))}[kind]
        past = int(rng.integers(0, 20001)) if rng.random() < 0.1 else int(rng.integers(0, 3001))
        if ql == 0:
            past = max(past, 1)
        lens.append(past + ql)
        qlens.append(ql)
    sc = float(rng.choice([2.0 ** -5, 0.05])) if kv == "fp8_e4m3" else 1.0
    return dict(lens=lens, qlens=qlens, num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=d, block_size=B,
                kv_dtype=kv, q_dtype=q, k_scale=sc, v_scale=sc * 1.5 if kv == "fp8_e4m3" else 1.0)


@pytest.mark.parametrize("seed", range(24))
def test_random_step(seed):
    spec = draw_step(seed)
    lens, qlens = spec.pop("lens"), spec.pop("qlens")
    label = (f"random seed={seed} n={len(lens)} max_len={max(lens)} tokens={sum(qlens)} "
             f"{spec['kv_dtype']}/{spec['q_dtype']} d={spec['head_dim']} B={spec['block_size']} "
             f"Hq={spec['num_q_heads']} Hkv={spec['num_kv_heads']}")
    say(label)
    w = build("random", 100 + seed, lens, qlens, **spec)
    kp, vp = oracle.cache.fill_pools(w)
    ref = oracle.attention.paged_attention(
        w.q_values(), w.q_dtype, kp, vp, w.kv_dtype, w.block_tables, w.seq_lens,
        w.query_start_loc, w.block_size, w.scale, w.k_scale, w.v_scale)
    step = wd.stage(w)
    out = step.attend()
    torch.cuda.synchronize()
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    if got.size == 0:
        return
    assert not np.isnan(got).any(), f"{label}: NaN in GPU output"
    err = float(np.abs(got - ref).max())
    say(f"  max-abs err {err:.3e} (tol {TOL[w.kv_dtype]:.0e}) over {got.size} values")
    assert err <= TOL[w.kv_dtype], f"{label}: max-abs error {err} > {TOL[w.kv_dtype]}"


@pytest.mark.parametrize("seed", range(100, 112))
def test_random_step_through_the_joint_call(seed):
    # the same draws through pa_write_and_attend (the new tokens' cache
    # write in the plan's launch): the whole pools byte for byte against the
    # oracle's cache write, every row against the oracle's attention
    spec = draw_step(seed)
    lens, qlens = spec.pop("lens"), spec.pop("qlens")
    label = (f"joint random seed={seed} n={len(lens)} max_len={max(lens)} tokens={sum(qlens)} "
             f"{spec['kv_dtype']}/{spec['q_dtype']} d={spec['head_dim']} B={spec['block_size']} "
             f"Hq={spec['num_q_heads']} Hkv={spec['num_kv_heads']}")
    say(label)
    w = build("random_joint", 100 + seed, lens, qlens, **spec)
    kp, vp = oracle.cache.fill_pools(w)
    ref = oracle.attention.paged_attention(
        w.q_values(), w.q_dtype, kp, vp, w.kv_dtype, w.block_tables, w.seq_lens,
        w.query_start_loc, w.block_size, w.scale, w.k_scale, w.v_scale)
    step = wd.stage(w, write_new=False)
    out = step.write_and_attend(out=torch.full_like(step.q, float("nan")))
    torch.cuda.synchronize()
    assert np.array_equal(wd.to_host_bits(step.k_cache), kp), f"{label}: K pool"
    assert np.array_equal(wd.to_host_bits(step.v_cache), vp), f"{label}: V pool"
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    if got.size == 0:
        return
    assert not np.isnan(got).any(), f"{label}: NaN in GPU output"
    err = float(np.abs(got - ref).max())
    say(f"  max-abs err {err:.3e} (tol {TOL[w.kv_dtype]:.0e}) over {got.size} values")
    assert err <= TOL[w.kv_dtype], f"{label}: max-abs error {err} > {TOL[w.kv_dtype]}"
