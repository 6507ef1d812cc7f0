"""pa_write_and_attend: the cache write of a step's new tokens and the
step's attention in one call, against the two separate calls on the same
inputs -- pools and output bit-exact -- and against the fp64 oracle."""

import numpy as np
import pytest

import workloads
from oracle import codecs
from workloads import device as wd
from workloads.generate import build, random_mixed

from full_oracle import assert_close, attention, fill_pools, say

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402,F401

pytestmark = pytest.mark.gpu


def _bits(t):
    return wd.to_host_bits(t).copy()


CASES = [
    ("tiny_decode", lambda: workloads.make("tiny_decode")),
    ("decode bf16, split tail, d 256", lambda: build("wa_split", 3, [9000, 14000, 11000, 9500], [1, 1, 2, 1],
                                                    num_q_heads=16, num_kv_heads=4, head_dim=256, block_size=16,
                                                    kv_dtype="bf16")),
    ("mixed bf16 (fused launch)", lambda: random_mixed(5, num_decode=20, chunk_specs=[(0, 100), (700, 300)],
                                                       max_decode_len=3000, num_q_heads=32, num_kv_heads=8,
                                                       head_dim=128, block_size=16, kv_dtype="bf16")),
    ("mixed fp8 from f32 rows", lambda: random_mixed(6, num_decode=12, chunk_specs=[(0, 80)], max_decode_len=2000,
                                                     num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=32,
                                                     kv_dtype="fp8_e4m3", src_dtype="f32", q_dtype="f16",
                                                     k_scale=2.0 ** -5, v_scale=2.0 ** -5)),
    ("mixed d 256 (kernels apart)", lambda: random_mixed(7, num_decode=8, chunk_specs=[(0, 70)], max_decode_len=1500,
                                                         num_q_heads=8, num_kv_heads=4, head_dim=256, block_size=64,
                                                         kv_dtype="f16")),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_joint_call_equals_two_calls(name, make):
    w = make()
    say(f"write_and_attend: {name}: {w.summary()}")
    # two calls
    a = wd.stage(w, write_new=False)
    a.write_new()
    ref = _bits(a.attend())
    ref_k, ref_v = _bits(a.k_cache), _bits(a.v_cache)
    # one call, on an identically staged pool
    b = wd.stage(w, write_new=False)
    out = torch.full_like(b.q, float("nan"))
    got = _bits(b.write_and_attend(out=out))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(b.k_cache), ref_k) and np.array_equal(_bits(b.v_cache), ref_v)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} of {got.size} elements differ"
    # and the oracle
    kp, vp = fill_pools(w)
    assert_close(w, codecs.decode(got, w.q_dtype), attention(w, kp, vp), label=f"write_and_attend {name}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_joint_call_with_a_shared_prefix(kv):
    # pa_write_and_attend with prefix_len > 0 against pa_reshape_and_cache +
    # pa_attention_shared_prefix
    P = 2048
    fp8 = kv == "fp8_e4m3"
    w = build("wa_prefix", 11, [P + 10, P + 700, P + 1, P + 333, P + 1500], [1, 1, 1, 2, 1], num_q_heads=16,
              num_kv_heads=4, head_dim=128, block_size=32, kv_dtype=kv, shared_prefix_len=P,
              k_scale=2.0 ** -5 if fp8 else 1.0, v_scale=2.0 ** -5 if fp8 else 1.0)
    a = wd.stage(w, write_new=False).use_shared_prefix(P)
    a.write_new()
    ref = _bits(a.attend())
    b = wd.stage(w, write_new=False).use_shared_prefix(P)
    got = _bits(b.write_and_attend(out=torch.full_like(b.q, float("nan"))))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(b.k_cache), _bits(a.k_cache)) and np.array_equal(_bits(b.v_cache), _bits(a.v_cache))
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} of {got.size} elements differ"
    kp, vp = fill_pools(w)
    assert_close(w, codecs.decode(got, w.q_dtype), attention(w, kp, vp), label=f"write_and_attend prefix {kv}")


def test_bound_call_equals_the_plain_call():
    # bind_write_and_attend marshals once and issues the same call: two
    # calls of the bound form give the plain call's pools and output
    w = build("wa_bound", 13, [700, 2300, 40], [1, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128,
              block_size=16, kv_dtype="bf16")
    a = wd.stage(w, write_new=False)
    ref = _bits(a.write_and_attend())
    b = wd.stage(w, write_new=False)
    run = b.bound_step()
    run()
    got = _bits(run())
    torch.cuda.synchronize()
    assert np.array_equal(got, ref)
    assert np.array_equal(_bits(b.k_cache), _bits(a.k_cache)) and np.array_equal(_bits(b.v_cache), _bits(a.v_cache))


def _tiny_bf16():
    return build("wa_edge", 21, [40, 300, 17, 1000], [1, 2, 1, 1], num_q_heads=8, num_kv_heads=2, head_dim=128,
                 block_size=16, kv_dtype="bf16")


def test_joint_call_with_nothing_to_write():
    # no new rows (null key/value/slot pointers, 0 tokens): the attention alone
    w = _tiny_bf16()
    a = wd.stage(w)
    ref = _bits(a.attend())
    b = wd.stage(w)
    e = b.new_key[:0]
    out = pa.write_and_attend(e, b.new_value[:0], b.new_slots[:0], b.q, b.k_cache, b.v_cache, b.block_tables,
                              b.seq_lens, b.query_start_loc, w.scale, max_seq_len=w.max_seq_len,
                              max_query_len=w.max_query_len, out=torch.full_like(b.q, float("nan")),
                              workspace=b.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), ref)
    assert np.array_equal(_bits(b.k_cache), _bits(a.k_cache)) and np.array_equal(_bits(b.v_cache), _bits(a.v_cache))


def test_joint_call_with_no_query_rows():
    # writes but an empty step (no sequences): the cache write alone
    w = _tiny_bf16()
    a = wd.stage(w, write_new=False)
    a.write_new()
    torch.cuda.synchronize()
    b = wd.stage(w, write_new=False)
    dev = b.q.device
    q0 = b.q[:0]
    out = pa.write_and_attend(b.new_key, b.new_value, b.new_slots, q0, b.k_cache, b.v_cache,
                              torch.zeros(0, b.block_tables.shape[1], dtype=torch.int32, device=dev),
                              torch.zeros(0, dtype=torch.int32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev),
                              w.scale, max_seq_len=w.max_seq_len, max_query_len=1, out=torch.empty_like(q0),
                              workspace=b.workspace)
    torch.cuda.synchronize()
    assert out.numel() == 0
    assert np.array_equal(_bits(b.k_cache), _bits(a.k_cache)) and np.array_equal(_bits(b.v_cache), _bits(a.v_cache))


def test_joint_call_skips_negative_slots():
    # rows whose slot is negative are not written, in the joint call as in
    # pa_reshape_and_cache: every other new row lands, the skipped slots keep
    # what the pool held (here the poison), and both calls give one output
    w = _tiny_bf16()
    a = wd.stage(w, write_new=False)
    b = wd.stage(w, write_new=False)
    slots = a.new_slots.clone()
    slots[1] = -1
    slots[3] = -7
    pa.reshape_and_cache(a.new_key, a.new_value, a.k_cache, a.v_cache, slots, w.k_scale, w.v_scale)
    ref = _bits(a.attend())
    out = pa.write_and_attend(b.new_key, b.new_value, slots, b.q, b.k_cache, b.v_cache, b.block_tables,
                              b.seq_lens, b.query_start_loc, w.scale, max_seq_len=w.max_seq_len,
                              max_query_len=w.max_query_len, out=torch.full_like(b.q, float("nan")),
                              workspace=b.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(b.k_cache), _bits(a.k_cache)) and np.array_equal(_bits(b.v_cache), _bits(a.v_cache))
    # NaN-poisoned skipped slots make NaN rows on both sides: compare bits
    assert np.array_equal(_bits(out), ref)
    kb = _bits(b.k_cache)
    s = int(a.new_slots[1].item())
    assert np.all(kb[s // w.block_size, :, s % w.block_size, :] == w.poison())


def _joint_against_oracle(w, prefix, label):
    import oracle
    kp, vp = oracle.cache.fill_pools(w)
    ref = oracle.attention.paged_attention(w.q_values(), w.q_dtype, kp, vp, w.kv_dtype, w.block_tables, w.seq_lens,
                                           w.query_start_loc, w.block_size, w.scale, w.k_scale, w.v_scale)
    step = wd.stage(w, write_new=False)
    if prefix:
        step.use_shared_prefix(prefix)
    out = step.write_and_attend(out=torch.full_like(step.q, float("nan")))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(step.k_cache), kp) and np.array_equal(_bits(step.v_cache), vp), f"{label}: pools"
    got = codecs.decode(_bits(out), w.q_dtype)
    tol = {"f32": 2e-3, "f16": 2e-3, "bf16": 1e-2, "fp8_e4m3": 4e-2}[w.kv_dtype]
    assert not np.isnan(got).any(), f"{label}: NaN"
    err = float(np.abs(got - ref).max())
    say(f"{label}: max-abs err {err:.2e} (tol {tol:.0e})")
    assert err <= tol, f"{label}: {err}"


@pytest.mark.parametrize("seed", range(6))
def test_random_shared_prefix_steps_through_the_joint_call(seed):
    # seeded cascade steps (prefix of whole blocks; per sequence a decode
    # token, a short run or a prompt chunk past it) with their cache write
    rng = np.random.default_rng([seed, 17])
    d = int(rng.choice([64, 128, 256]))
    B = int(rng.choice([16, 32, 64]))
    kv = str(rng.choice(["f16", "bf16", "fp8_e4m3"]))
    q = {"f16": "f16", "bf16": "bf16"}.get(kv) or str(rng.choice(["bf16", "f16"]))
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    P = B * int(rng.integers(1, 6000 // B))
    n = int(rng.integers(1, 13))
    qlens = [int(rng.choice([1, 1, 1, int(rng.integers(2, 9)), int(rng.integers(16, 160))])) for _ in range(n)]
    lens = [P + ql + int(rng.integers(0, 1200)) for ql in qlens]
    sc = float(rng.choice([2.0 ** -5, 0.05])) if kv == "fp8_e4m3" else 1.0
    w = build("wa_pfx_rand", 500 + seed, lens, qlens, num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=d,
              block_size=B, kv_dtype=kv, q_dtype=q, k_scale=sc, v_scale=sc, shared_prefix_len=P)
    _joint_against_oracle(w, P, f"joint cascade seed={seed} {kv}/{q} d={d} B={B} G={G} Hkv={hkv} P={P} n={n}")


@pytest.mark.parametrize("seed", range(6))
def test_random_fused_mixed_steps_through_the_joint_call(seed):
    # seeded mixed steps that take the fused launch (16-bit q, head dim <= 128,
    # prompt chunks of at least 65 rows per kv head) with their cache write
    rng = np.random.default_rng([seed, 19])
    d = int(rng.choice([64, 128]))
    B = int(rng.choice([16, 32, 64]))
    kv = str(rng.choice(["f16", "bf16", "fp8_e4m3"]))
    q = {"f16": "f16", "bf16": "bf16"}.get(kv) or str(rng.choice(["bf16", "f16"]))
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    chunks = [(int(rng.integers(0, 8000)), int(rng.integers(-(-65 // G), 400))) for _ in range(int(rng.integers(1, 4)))]
    sc = float(rng.choice([2.0 ** -5, 0.05])) if kv == "fp8_e4m3" else 1.0
    w = random_mixed(600 + seed, num_decode=int(rng.integers(1, 120)), chunk_specs=chunks,
                     max_decode_len=int(rng.integers(10, 5000)), num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=d,
                     block_size=B, kv_dtype=kv, q_dtype=q, k_scale=sc, v_scale=sc, name="wa_mixed_rand")
    _joint_against_oracle(w, 0, f"joint fused seed={seed} {kv}/{q} d={d} B={B} G={G} Hkv={hkv} chunks={chunks}")
