"""GPU parity of the fused step kernel: a step that can hold prompt chunks
(16-bit q, head dim <= 128) runs its decode and chunk items in one launch,
split between the two lists by the plan kernel.  These cases push the split
to its ends (no decode items, no chunk items, a host hint that overstates the
longest query) and through a step with many more chunk rows than decode rows,
each against the fp64 oracle."""

import sys

import numpy as np
import pytest

import oracle
from oracle import codecs
from workloads import device as wd
from workloads.generate import build, random_mixed

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-3, "f16": 2e-3, "bf16": 1e-2, "fp8_e4m3": 4e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def oracle_out(w):
    kp, vp = oracle.cache.fill_pools(w, None)
    return oracle.attention.paged_attention(
        w.q_values(), w.q_dtype, kp, vp, w.kv_dtype, w.block_tables, w.seq_lens,
        w.query_start_loc, w.block_size, w.scale, w.k_scale, w.v_scale)


def check(w, out, label):
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    ref = oracle_out(w)
    assert not np.isnan(got).any(), f"{label}: NaN"
    err = float(np.abs(got - ref).max())
    say(f"{label}: max-abs err {err:.3e} (tol {TOL[w.kv_dtype]:.0e})")
    assert err <= TOL[w.kv_dtype], f"{label}: {err}"


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_chunks_only(kv):
    # prompt chunks and no decode row: every workgroup takes chunk items
    sc = 0.05 if kv == "fp8_e4m3" else 1.0
    w = build("chunks_only", 41, [700, 300, 1500], [700, 200, 130], num_q_heads=8, num_kv_heads=2,
              head_dim=128, block_size=16, kv_dtype=kv, q_dtype="bf16", k_scale=sc, v_scale=sc)
    say("chunks_only", kv)
    st = wd.stage(w)
    check(w, st.attend(), f"chunks_only {kv}")


def test_decode_rows_with_overstated_hint():
    # decode rows only, but the host hint allows prompt chunks: the fused
    # launch runs with an empty chunk list and every workgroup on decode items
    w = random_mixed(43, num_decode=40, chunk_specs=[], max_decode_len=3000, num_q_heads=16,
                     num_kv_heads=4, head_dim=128, block_size=16, kv_dtype="bf16")
    say("decode_overstated_hint")
    st = wd.stage(w)
    out = pa.attention(st.q, st.k_cache, st.v_cache, st.block_tables, st.seq_lens, st.query_start_loc,
                       w.scale, max_seq_len=w.max_seq_len, max_query_len=64)
    check(w, out, "decode, max_query_len hint 64")


@pytest.mark.parametrize("kv,d", [("bf16", 64), ("f16", 128), ("fp8_e4m3", 128)])
def test_mixed_split(kv, d):
    # many decode rows beside chunks of several lengths and offsets
    sc = 0.05 if kv == "fp8_e4m3" else 1.0
    q = "f16" if kv == "f16" else "bf16"
    w = random_mixed(47, num_decode=120, chunk_specs=[(0, 128), (500, 200), (1000, 70)], max_decode_len=1200,
                     num_q_heads=8, num_kv_heads=2, head_dim=d, block_size=16, kv_dtype=kv, q_dtype=q,
                     k_scale=sc, v_scale=sc)
    say("mixed_split", kv, d)
    st = wd.stage(w)
    check(w, st.attend(), f"mixed_split {kv} d={d}")


def test_fused_replays_bit_exact():
    # the split and the lists are rebuilt every call; outputs must not move
    w = random_mixed(53, num_decode=64, chunk_specs=[(100, 300)], max_decode_len=2000, num_q_heads=8,
                     num_kv_heads=2, head_dim=128, block_size=16, kv_dtype="bf16")
    st = wd.stage(w)
    first = wd.to_host_bits(st.attend()).copy()
    for _ in range(3):
        assert np.array_equal(first, wd.to_host_bits(st.attend()))


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_mixed_step_graph_replays_bit_exact(kv):
    # one mixed step (cache write of the new tokens, plan, fused kernel,
    # merge) captured in a HIP graph; each replay, with eager library work
    # and a poisoned output in between, must reproduce the eager output
    sc = 2.0 ** -5 if kv == "fp8_e4m3" else 1.0
    w = random_mixed(61, num_decode=48, chunk_specs=[(0, 200), (300, 150), (9000, 100)], max_decode_len=3000,
                     num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, kv_dtype=kv, q_dtype="bf16",
                     k_scale=sc, v_scale=sc)
    say("mixed_graph", kv)
    st = wd.stage(w, write_new=False)
    out = st.step()
    torch.cuda.synchronize()
    eager = wd.to_host_bits(out).copy()
    check(w, out, f"mixed_graph eager {kv}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step()
    for rep in range(3):
        st.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(wd.to_host_bits(st.out), eager), f"replay {rep} differs from the eager step"
        st.attend()                                  # eager work between replays
        torch.cuda.synchronize()
