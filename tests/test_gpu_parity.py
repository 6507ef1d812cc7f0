"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Cache writes must match the oracle byte for byte; attention must be within
max-abs 2e-3 (fp32/fp16 KV), 1e-2 (bf16 KV) or 4e-2 (fp8 KV) of the oracle,
with no NaN.  Invariants (placement permutation, shared vs private prefix
blocks, run-to-run) must hold bit-exactly on the GPU.
"""

import numpy as np
import pytest

import oracle
import workloads
from oracle import codecs
from workloads import device as wd
from workloads.generate import build, random_mixed

from full_oracle import TOL, assert_close, attention, fill_pools, rows_of, say  # noqa: F401

torch = pytest.importorskip("torch")
import paged_kv_cache_141_amd as pa  # noqa: E402

pytestmark = pytest.mark.gpu


def oracle_out(w, seqs=None):
    kp, vp = fill_pools(w, seqs)
    return attention(w, kp, vp, seqs)


def gpu_out(step):
    out = step.attend()
    torch.cuda.synchronize()
    return codecs.decode(wd.to_host_bits(out), step.w.q_dtype)


def timed_call_out(w, prefix=0, calls=2):
    """The step as the throughput measurement issues it: the new tokens'
    cache write and the attention in one pa_write_and_attend call, arguments
    marshalled once, called ``calls`` times (a repeat writes the same bytes).
    Checks the new tokens' slots byte for byte; returns the decoded output."""
    step = wd.stage(w, write_new=False)
    if prefix:
        step.use_shared_prefix(prefix)
    run = step.bound_step()
    for _ in range(calls):
        out = run()
    torch.cuda.synchronize()
    kbits, vbits = wd.to_host_bits(step.k_cache), wd.to_host_bits(step.v_cache)
    nk, nv, ns = w.new_token_batch()
    blk, off = ns // w.block_size, ns % w.block_size
    # the oracle's encoding of the new rows (bf16 into fp8 caches)
    ek = oracle.cache.encode_tokens(nk, w.src_dtype, w.kv_dtype, w.k_scale)
    ev = oracle.cache.encode_tokens(nv, w.src_dtype, w.kv_dtype, w.v_scale)
    assert np.array_equal(kbits[blk, :, off, :], ek), "new K rows"
    assert np.array_equal(vbits[blk, :, off, :], ev), "new V rows"
    got = codecs.decode(wd.to_host_bits(out), w.q_dtype)
    del step, kbits, vbits
    torch.cuda.empty_cache()
    return got


# ------------------------------------------------------------------ cache write

SPECIAL_F32 = np.array([0.0, -0.0, 1.0, -1.5, 3.0e38, -3.4e38, np.inf, -np.inf, np.nan, 1e-40,
                        -1e-45, 6e-8, 65504.0, 65520.0, 70000.0, 448.0, 464.0, 480.0, -1e6,
                        1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -11, 2 ** -10, 3 * 2 ** -10,
                        2 ** -7 * 1.0625, 0.0009765625, 5.9604645e-08, 2.9802322e-08],
                       dtype=np.float32)


def _src_values(shape, src, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * 4).astype(np.float32)
    flat = x.reshape(-1)
    flat[:SPECIAL_F32.size] = SPECIAL_F32
    flat[-SPECIAL_F32.size:] = SPECIAL_F32[::-1] * np.float32(0.37)
    if src == "f32":
        return x
    if src == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)        # bf16 bits


@pytest.mark.parametrize("src,kv,B,d,scale", [
    ("f32", "f32", 16, 64, 1.0), ("bf16", "bf16", 16, 128, 1.0), ("f16", "f16", 32, 64, 1.0),
    ("f32", "bf16", 16, 128, 1.0), ("f32", "f16", 64, 128, 1.0), ("bf16", "f16", 16, 64, 1.0),
    ("bf16", "fp8_e4m3", 16, 128, 2.0 ** -5), ("bf16", "fp8_e4m3", 64, 128, 0.0123),
    ("f32", "fp8_e4m3", 32, 64, 0.37), ("f16", "fp8_e4m3", 16, 64, 1.0),
    ("bf16", "bf16", 32, 256, 1.0), ("f32", "fp8_e4m3", 16, 256, 0.05)])
@pytest.mark.parametrize("runs", [False, True])
def test_cache_write_bit_exact(src, kv, B, d, scale, runs):
    say(f"cache write {src}->{kv} B={B} d={d} scale={scale} runs={runs}")
    H, T, N = 3, 77, 24
    w = build("cw", 5, [T], [T], num_q_heads=H, num_kv_heads=H, head_dim=d, block_size=B,
              kv_dtype=kv, src_dtype=src, q_dtype="bf16" if kv != "f32" else "f32",
              k_scale=scale if kv == "fp8_e4m3" else 1.0, v_scale=scale / 3 if kv == "fp8_e4m3" else 1.0,
              num_blocks=N)
    key = _src_values((T, H, d), src, 1)
    val = _src_values((T, H, d), src, 2)
    rng = np.random.default_rng(3)
    if runs:
        # a prompt chunk: consecutive slots through shuffled blocks, starting
        # mid-block, with a stretch of padding
        order = rng.permutation(N)
        start = B // 2 + 3
        slots = np.array([order[(start + t) // B] * B + (start + t) % B for t in range(T)], dtype=np.int64)
        slots[40:45] = -1
    else:
        slots = rng.permutation(N * B)[:T].astype(np.int64)
        slots[::7] = -1                                 # padding tokens are skipped
    kp, vp = w.initial_pool()
    oracle.cache.reshape_and_cache(kp, vp, key, val, src, kv, slots, B, w.k_scale, w.v_scale)
    kc, vc = wd.poisoned_pool(w, "cuda")
    pa.reshape_and_cache(wd.to_device(key, src, "cuda"), wd.to_device(val, src, "cuda"), kc, vc,
                         torch.from_numpy(slots).cuda(), w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    gk, gv = wd.to_host_bits(kc), wd.to_host_bits(vc)
    bad_k = np.argwhere(gk != kp)
    bad_v = np.argwhere(gv != vp)
    assert bad_k.size == 0, f"K differs at {bad_k[:5].tolist()}: gpu {gk[tuple(bad_k[0])]:#x} oracle {kp[tuple(bad_k[0])]:#x}"
    assert bad_v.size == 0, f"V differs at {bad_v[:5].tolist()}"


# ------------------------------------------------------------------ attention, small

SMALL = [
    # kv, q, B, d, Hq, Hkv, chunks
    ("f32", "f32", 16, 64, 2, 2, []),
    ("f32", "f32", 32, 128, 8, 2, [(0, 40), (70, 33)]),
    ("bf16", "bf16", 16, 128, 32, 8, [(0, 24), (100, 50)]),
    ("bf16", "bf16", 32, 64, 4, 4, [(0, 64), (33, 17)]),
    ("bf16", "bf16", 64, 128, 16, 2, [(5, 30)]),
    ("f16", "f16", 16, 128, 8, 8, [(0, 21)]),
    ("f16", "f16", 64, 64, 6, 2, [(12, 31)]),                 # G = 3
    ("fp8_e4m3", "bf16", 16, 128, 32, 8, [(0, 40)]),
    ("fp8_e4m3", "bf16", 32, 128, 16, 1, [(9, 9)]),           # G = 16
    ("fp8_e4m3", "f16", 64, 64, 8, 4, [(0, 3), (200, 20)]),
    ("bf16", "bf16", 16, 256, 16, 4, [(0, 40), (90, 30)]),       # head dim 256: one step in flight,
    ("f16", "f16", 32, 256, 8, 8, [(3, 70)]),                   # 128-row chunk items
    ("fp8_e4m3", "bf16", 64, 256, 8, 2, [(0, 64), (130, 17)]),
    ("fp8_e4m3", "f16", 16, 256, 8, 4, [(0, 20)]),
    ("bf16", "bf16", 64, 256, 4, 4, [(5, 30)]),
]


@pytest.mark.parametrize("kv,q,B,d,Hq,Hkv,chunks", SMALL)
def test_attention_small(kv, q, B, d, Hq, Hkv, chunks):
    label = f"small kv={kv} q={q} B={B} d={d} Hq={Hq} Hkv={Hkv} chunks={chunks}"
    say(label)
    fp8 = kv == "fp8_e4m3"
    w = random_mixed(17, num_decode=9, chunk_specs=chunks, max_decode_len=1400, num_q_heads=Hq,
                     num_kv_heads=Hkv, head_dim=d, block_size=B, kv_dtype=kv, q_dtype=q,
                     k_scale=2.0 ** -5 if fp8 else 1.0, v_scale=1.5 * 2.0 ** -5 if fp8 else 1.0)
    step = wd.stage(w)
    assert_close(w, gpu_out(step), oracle_out(w), label=label)


def test_tiny_decode():
    w = workloads.make("tiny_decode")
    say("tiny_decode", w.summary())
    step = wd.stage(w)
    assert_close(w, gpu_out(step), oracle_out(w), label="tiny_decode")


def test_edge_lengths():
    # L = 1, lengths at block/step/partition boundaries, a q_len = 0 sequence,
    # a chunk that is the whole prompt, and a length past one 512-key partition.
    lens = [1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1024, 1025, 7, 300]
    qlens = [1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 300]
    for kv, q, B in (("bf16", "bf16", 16), ("fp8_e4m3", "bf16", 64), ("f32", "f32", 32)):
        sc = 0.05 if kv == "fp8_e4m3" else 1.0
        w = build("edge", 23, lens, qlens, num_q_heads=8, num_kv_heads=2, head_dim=128,
                  block_size=B, kv_dtype=kv, q_dtype=q, k_scale=sc, v_scale=sc)
        say("edge", kv, B)
        step = wd.stage(w)
        assert_close(w, gpu_out(step), oracle_out(w), label=f"edge {kv} B={B}")


def test_edge_lengths_long_context():
    # A step whose longest context passes 8192 keys, with 14 x 16 (sequence,
    # kv head) pairs, splits decode rows into 1024-key partitions: lengths at
    # those boundaries, a decode row one partition long, and a prompt chunk
    # that crosses the chunk kernel's 8192-key partition boundary.
    lens = [1, 1023, 1024, 1025, 2047, 2048, 2049, 4097, 8191, 8192, 8193, 12000, 8300, 9000]
    qlens = [1] * 12 + [200, 1]
    for kv, q, B in (("bf16", "bf16", 16), ("fp8_e4m3", "bf16", 32), ("f32", "f32", 64)):
        sc = 0.05 if kv == "fp8_e4m3" else 1.0
        w = build("edge_long", 29, lens, qlens, num_q_heads=32, num_kv_heads=16, head_dim=64,
                  block_size=B, kv_dtype=kv, q_dtype=q, k_scale=sc, v_scale=sc)
        say("edge_long", kv, B)
        step = wd.stage(w)
        assert_close(w, gpu_out(step), oracle_out(w), label=f"edge_long {kv} B={B}")


def test_edge_lengths_fused_partition():
    # 16-bit q with chunks runs the fused step, whose chunk items cover
    # 16384-key partitions (8192 for f32, kernels apart): prompt chunks whose
    # rows straddle key 16384 and 8192, one that ends on 16384, and decode
    # rows at the boundary.
    lens = [16500, 16384, 16385, 16383, 8300, 20000, 1, 16448]
    qlens = [300, 1, 1, 64, 200, 1, 1, 64]
    for kv, q, B in (("bf16", "bf16", 16), ("fp8_e4m3", "f16", 32), ("f32", "f32", 16)):
        sc = 0.05 if kv == "fp8_e4m3" else 1.0
        w = build("edge_fused", 37, lens, qlens, num_q_heads=8, num_kv_heads=4, head_dim=64,
                  block_size=B, kv_dtype=kv, q_dtype=q, k_scale=sc, v_scale=sc)
        say("edge_fused", kv, B)
        step = wd.stage(w)
        assert_close(w, gpu_out(step), oracle_out(w), label=f"edge_fused {kv} B={B}")


def test_edge_lengths_many_pairs():
    # 256 sequences x 8 kv heads: enough (sequence, kv head) pairs for
    # 2048-key decode partitions (128 blocks of 16 keys: block ids in two
    # registers per lane): lengths at those boundaries, and a prompt chunk
    # that crosses one.
    rng = np.random.default_rng([31, 0])
    edges = [1, 63, 64, 65, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097, 6000]
    lens = edges + [int(x) for x in rng.integers(1, 400, size=255 - len(edges))] + [2300]
    qlens = [1] * 255 + [100]
    for kv, q, B in (("bf16", "bf16", 16), ("fp8_e4m3", "bf16", 32), ("f32", "f32", 64)):
        sc = 0.05 if kv == "fp8_e4m3" else 1.0
        w = build("edge_pairs", 31, lens, qlens, num_q_heads=16, num_kv_heads=8, head_dim=64,
                  block_size=B, kv_dtype=kv, q_dtype=q, k_scale=sc, v_scale=sc)
        say("edge_pairs", kv, B)
        step = wd.stage(w)
        assert_close(w, gpu_out(step), oracle_out(w), label=f"edge_pairs {kv} B={B}")


@pytest.mark.parametrize("chunks", [False, True])
def test_many_sequences(chunks):
    # 2,500 sequences: the plan takes sequences 1,024 at a time, and the merge
    # finds a token's sequence by binary search over all of them; with prompt
    # chunks among them the step runs the fused launch
    specs = [(40, 100), (0, 70), (900, 80)] if chunks else []
    w = random_mixed(59, num_decode=2500 - len(specs), chunk_specs=specs, max_decode_len=1100, num_q_heads=4,
                     num_kv_heads=2, head_dim=64, block_size=16, kv_dtype="bf16")
    say("many_sequences", w.num_seqs, "chunks" if chunks else "decode only")
    step = wd.stage(w)
    assert_close(w, gpu_out(step), oracle_out(w), label=f"many_sequences chunks={chunks}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_very_long_context(kv):
    # contexts of 128k tokens and more: 129 decode partitions of 1024 keys for one row, a
    # prompt chunk 100,000 keys in (13 chunk partitions), partials merged
    sc = 0.05 if kv == "fp8_e4m3" else 1.0
    lens = [131077, 100100, 40000, 9]
    qlens = [1, 100, 1, 1]
    w = build("very_long", 61, lens, qlens, num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=16,
              kv_dtype=kv, q_dtype="bf16", k_scale=sc, v_scale=sc)
    say("very_long", kv, w.max_seq_len)
    step = wd.stage(w)
    assert_close(w, gpu_out(step), oracle_out(w), label=f"very_long {kv}")


# ------------------------------------------------------------------ invariants

def test_placement_permutation_bit_exact():
    a = wd.stage(workloads.make("llama7b_decode", num_seqs=24))
    b = wd.stage(workloads.make("llama7b_decode", num_seqs=24, placement="identity"))
    oa, ob = wd.to_host_bits(a.attend()), wd.to_host_bits(b.attend())
    assert np.array_equal(oa, ob)


def test_shared_prefix_equals_private_bit_exact():
    s = wd.stage(workloads.make("fp8_shared_prefix", num_seqs=8))
    p = wd.stage(workloads.make("fp8_shared_prefix", num_seqs=8, placement="private"))
    assert np.array_equal(wd.to_host_bits(s.attend()), wd.to_host_bits(p.attend()))


def test_deterministic_run_to_run():
    st = wd.stage(workloads.make("gqa_long_decode", num_seqs=6))
    first = wd.to_host_bits(st.attend()).copy()
    for _ in range(3):
        assert np.array_equal(first, wd.to_host_bits(st.attend()))


def test_metadata_checker():
    w = workloads.make("tiny_decode")
    st = wd.stage(w)
    ok, bad = pa.check_metadata(st.k_cache, st.v_cache, st.block_tables, st.seq_lens,
                                st.query_start_loc, w.num_tokens, w.max_seq_len, w.max_query_len)
    assert ok and bad == -1
    bt = st.block_tables.clone()
    bt[2, 0] = w.num_blocks
    ok, bad = pa.check_metadata(st.k_cache, st.v_cache, bt, st.seq_lens, st.query_start_loc,
                                w.num_tokens, w.max_seq_len, w.max_query_len)
    assert not ok and bad == 2
    lens = st.seq_lens.clone()
    lens[1] = 0                                   # q_len 1 > L 0
    ok, bad = pa.check_metadata(st.k_cache, st.v_cache, st.block_tables, lens, st.query_start_loc,
                                w.num_tokens, w.max_seq_len, w.max_query_len)
    assert not ok and bad == 1


# ------------------------------------------------------------------ full sizes, every row
#
# Each configuration at its full size, every query row against the oracle
# (the block-wise sum equals ordinary attention: itwiki "vLLM",
# "Block-wise attention"), through the call and launches the throughput
# measurement times (timed_call_out), with the step's cache write checked
# byte for byte at every new slot.

def test_full_llama7b_decode():
    w = workloads.make("llama7b_decode")
    say("full llama7b_decode: staging", w.summary())
    got = timed_call_out(w)
    kp, vp = fill_pools(w)
    assert_close(w, got, attention(w, kp, vp), label="llama7b_decode, every row")


def test_full_gqa_long_decode():
    w = workloads.make("gqa_long_decode")
    say("full gqa_long_decode: staging", w.summary())
    got = timed_call_out(w)
    kp, vp = fill_pools(w)
    assert_close(w, got, attention(w, kp, vp), label="gqa_long_decode, every row")


def test_full_mixed_chunked_prefill():
    w = workloads.make("mixed_chunked_prefill")
    say("full mixed_chunked_prefill: staging", w.summary())
    got = timed_call_out(w)                   # cache write of all new tokens + attention
    kp, vp = fill_pools(w)
    ref = attention(w, kp, vp)
    # the 1,024-token chunk at offset 8,192 (most of the chunk work) on its own line
    assert_close(w, got, ref, [258], label="mixed step, chunk at offset 8192")
    assert_close(w, got, ref, label="mixed step (decode + chunks), every row")


@pytest.mark.parametrize("B", [16, 32, 64])
def test_full_fp8_shared_prefix(B):
    # through the block tables (pa_attention) and through the shared-prefix
    # entry point (pa_attention_shared_prefix), both against the oracle
    w = workloads.make("fp8_shared_prefix", block_size=B)
    say(f"full fp8_shared_prefix B={B}: staging", w.summary())
    got = timed_call_out(w)
    cascade = timed_call_out(w, prefix=w.shared_prefix_len)
    kp, vp = fill_pools(w)
    ref = attention(w, kp, vp)
    assert_close(w, got, ref, label=f"fp8 shared prefix B={B} through the tables, every row")
    assert_close(w, cascade, ref, label=f"fp8 shared prefix B={B} through the cascade, every row")


def test_full_fp8_private_prefix_equals_shared():
    # The private-copy twin (each sequence owns copies of the prefix blocks)
    # gives bit for bit the output of the shared blocks, every row, so it meets
    # the oracle exactly where the shared case does (test above).
    shared = timed_call_out(workloads.make("fp8_shared_prefix", block_size=16))
    w = workloads.make("fp8_shared_prefix", block_size=16, placement="private")
    say("full fp8_private_prefix B=16: staging", w.summary())
    private = timed_call_out(w)
    assert np.array_equal(shared.view(np.uint64), private.view(np.uint64))


def test_decode_tiles_past_16_bits():
    # fp32 q keeps every row on the decode kernel, whose work items carry the
    # 16-row tile index in 16 unsigned bits.  An 8,200-token prompt with 64 q
    # heads on one kv head has 524,800 (token, head) rows = 32,800 tiles: the
    # tiles of tokens 8,192 on sit past 2^15.  Rows on both sides of that line
    # and a decode row are compared with the oracle.
    w = build("tiles16", 71, [8200, 300], [8200, 1], num_q_heads=64, num_kv_heads=1, head_dim=64,
              block_size=16, kv_dtype="f32", q_dtype="f32")
    say("tiles past 2^15:", w.summary())
    got = gpu_out(wd.stage(w))
    kp, vp = fill_pools(w)
    toks = np.r_[0:3, 4000:4003, 8100:8200]
    K, V = oracle.attention.gather_sequence(kp, vp, w.kv_dtype, 1.0, 1.0, w.block_tables[0], 8200, w.block_size)
    qf = codecs.decode(w.q_values(), w.q_dtype)
    ref = np.full(qf.shape, np.nan)
    ref[toks] = oracle.attention.attend_rows(qf[toks], K, V, toks, w.scale)   # positions = token index
    ref[8200:] = attention(w, kp, vp, [1])[8200:]
    sel = np.r_[toks, 8200]
    g, r = got[sel], ref[sel]
    assert not np.isnan(g).any()
    err = float(np.abs(g - r).max())
    say(f"tiles past 2^15: max-abs err {err:.3e} over {g.size} values")
    assert err <= TOL["f32"]


PAIRS = [("bf16", "bf16"), ("f16", "f16"), ("fp8_e4m3", "bf16"), ("fp8_e4m3", "f16"), ("f32", "f32")]


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("kv,q", PAIRS)
@pytest.mark.parametrize("G", [1, 4])
def test_attention_at_preferred_block_size(kv, q, d, G):
    # the pool sized with the block size the library recommends for this head
    # dim, precision and query group: a mixed step at that block size against
    # the oracle
    if d == 256 and q == "f32":
        pytest.skip("head dim 256 takes 16-bit queries only")
    code = {"f32": pa.PA_F32, "f16": pa.PA_F16, "bf16": pa.PA_BF16, "fp8_e4m3": pa.PA_FP8_E4M3}
    B = pa.preferred_block_size(d, code[kv], code[q], G)
    label = f"preferred B={B} for kv={kv} q={q} d={d} G={G}"
    say(label)
    fp8 = kv == "fp8_e4m3"
    w = random_mixed(400 + d + G, num_decode=11, chunk_specs=[(0, 70), (300, 45)], max_decode_len=2500,
                     num_q_heads=4 * G, num_kv_heads=4, head_dim=d, block_size=B, kv_dtype=kv, q_dtype=q,
                     k_scale=2.0 ** -5 if fp8 else 1.0, v_scale=2.0 ** -5 if fp8 else 1.0)
    assert_close(w, gpu_out(wd.stage(w)), oracle_out(w), label=label)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_long_context_mixed_step(kv):
    # decode rows at 20k-33k contexts beside two 512-token prompt chunks deep
    # into 20k-token prompts: few sequences, many chunk tokens, so decode rows
    # keep their partials in per-sequence slots and only chunk rows pay for
    # the long contexts at the chunk partition length (the split layout)
    sc = 2.0 ** -5 if kv == "fp8_e4m3" else 1.0
    lens = [20000, 24000, 28000, 33000, 21000, 30500, 20480, 19999]
    qlens = [1, 1, 1, 1, 1, 1, 512, 512]
    w = build("long_mixed", 97, lens, qlens, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
              kv_dtype=kv, q_dtype="bf16", k_scale=sc, v_scale=sc)
    lib = pa.library()
    import ctypes
    spec = pa._Cache(w.num_blocks, 16, 8, 128, pa.PA_BF16 if kv == "bf16" else pa.PA_FP8_E4M3, sc, sc)
    split, shared = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.pa_attention_workspace_size(ctypes.byref(spec), 32, w.num_seqs, w.num_tokens, w.max_seq_len,
                                           w.max_query_len, ctypes.byref(split)) == 0
    say(f"long mixed {kv}: {w.num_tokens} tokens, workspace {split.value / 2 ** 20:.1f} MiB "
        f"(token-indexed lists alone: {w.num_tokens * 32 * 17 * 520 / 2 ** 20:.1f} MiB)")
    assert split.value < w.num_tokens * 32 * 17 * 520          # smaller than one list per token
    got = gpu_out(wd.stage(w))
    assert_close(w, got, oracle_out(w), label=f"long-context mixed step {kv}")
