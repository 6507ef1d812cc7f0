"""Pins for the attention oracle and the cache-write oracle (CPU only).

The oracle is pinned to what the pages and the mathematics fix:
* the block-wise formula (itwiki "vLLM", "Block-wise attention") equals the
  gathered ordinary attention;
* a pure-Python brute force on the tiny decode shape;
* torch's scaled_dot_product_attention (a library routine) in float64;
* closed forms (one key, zero query, identical keys, a dominant key);
* invariants the pages state: physical placement does not matter (blocks need
  not be contiguous, "Block table"), shared blocks act like private copies
  ("Block sharing and copy-on-write"), chunked prefill gives the rows of the
  whole prompt ("Dynamic Chunked Prefill"), block size does not change the
  result;
* the log-sum-exp merge of context partitions reproduces the full softmax.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import cache as C
from oracle import codecs
import workloads
from workloads.generate import build


def run_oracle(w, seqs=None, form="gather"):
    kp, vp = C.fill_pools(w)
    fn = A.paged_attention if form == "gather" else A.block_sum_attention
    return fn(w.q_values(), w.q_dtype, kp, vp, w.kv_dtype, w.block_tables, w.seq_lens,
              w.query_start_loc, w.block_size, w.scale, w.k_scale, w.v_scale, seqs=seqs)


def small_mixed(kv_dtype="f32", q_dtype=None, placement="shuffled", B=16, seed=9, G=2):
    return workloads.generate.random_mixed(
        seed, num_decode=5, chunk_specs=[(0, 20), (17, 9), (40, 1)], max_decode_len=70,
        num_q_heads=2 * G, num_kv_heads=2, head_dim=32, block_size=B, kv_dtype=kv_dtype,
        q_dtype=q_dtype, k_scale=(2.0 ** -5 if kv_dtype == "fp8_e4m3" else 1.0),
        v_scale=(2.0 ** -5 if kv_dtype == "fp8_e4m3" else 1.0), placement=placement)


# ------------------------------------------------------------------ formula

@pytest.mark.parametrize("kv", ["f32", "bf16", "f16", "fp8_e4m3"])
def test_block_sum_formula_equals_gathered_attention(kv):
    w = small_mixed(kv)
    o1 = run_oracle(w)
    o2 = run_oracle(w, form="block")
    assert not np.isnan(o1).any()
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


def test_bruteforce_python_loops_tiny_decode():
    w = workloads.make("tiny_decode")
    out = run_oracle(w)
    kp, vp = C.fill_pools(w)
    q = w.q_values().astype(np.float64)
    B, d = w.block_size, w.head_dim
    kflat = kp.view(np.float32)
    vflat = vp.view(np.float32)
    for i in range(w.num_seqs):
        L = int(w.seq_lens[i])
        t = int(w.query_start_loc[i])
        for h in range(w.num_q_heads):
            g = h // w.group
            scores = []
            for pos in range(L):
                blk = int(w.block_tables[i][pos // B])
                off = pos % B
                s = sum(float(q[t, h, e]) * float(kflat[blk, g, off, e]) for e in range(d))
                scores.append(s * w.scale)
            m = max(scores)
            ws = [math.exp(s - m) for s in scores]
            tot = sum(ws)
            for e in range(d):
                acc = 0.0
                for pos in range(L):
                    blk = int(w.block_tables[i][pos // B])
                    acc += ws[pos] * float(vflat[blk, g, pos % B, e])
                assert abs(acc / tot - out[t, h, e]) < 1e-12


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8_e4m3"])
def test_matches_torch_sdpa_float64(kv):
    w = small_mixed(kv, G=4)
    out = run_oracle(w)
    kp, vp = C.fill_pools(w)
    qf = codecs.decode(w.q_values(), w.q_dtype)
    qsl = w.query_start_loc
    for i in range(w.num_seqs):
        L = int(w.seq_lens[i])
        a, b = int(qsl[i]), int(qsl[i + 1])
        n = b - a
        # independent gather: slot by slot through the table
        K = np.zeros((L, w.num_kv_heads, w.head_dim))
        V = np.zeros((L, w.num_kv_heads, w.head_dim))
        for pos in range(L):
            blk, off = int(w.block_tables[i][pos // w.block_size]), pos % w.block_size
            K[pos] = codecs.decode(kp[blk, :, off, :], w.kv_dtype) * w.k_scale
            V[pos] = codecs.decode(vp[blk, :, off, :], w.kv_dtype) * w.v_scale
        qt = torch.from_numpy(qf[a:b]).permute(1, 0, 2)                     # [Hq][n][d]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(w.group, 0)
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(w.group, 0)
        mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=w.scale).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[a:b], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ closed forms

def _single_seq(L, q_len=1, d=16, H=1, kv="f32", seed=1):
    return build("t", seed, [L], [q_len], num_q_heads=H, num_kv_heads=H, head_dim=d,
                 block_size=16, kv_dtype=kv)


def _attend(q, K, V, scale=0.25):
    pos = np.array([K.shape[0] - 1])
    return A.attend_rows(q[None, None, :], K[:, None, :], V[:, None, :], pos, scale)[0, 0]


def test_closed_form_single_key_returns_its_value():
    w = _single_seq(1)
    out = run_oracle(w)
    k, v = w.kv_values(0)
    assert np.array_equal(out[0, 0], v[0, 0].astype(np.float64))


def test_closed_form_zero_query_is_mean_of_values():
    rng = np.random.default_rng(0)
    K, V = rng.standard_normal((37, 8)), rng.standard_normal((37, 8))
    o = _attend(np.zeros(8), K, V)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-14)


def test_closed_form_identical_keys_is_mean_of_values():
    rng = np.random.default_rng(1)
    k = rng.standard_normal(8)
    K, V = np.tile(k, (21, 1)), rng.standard_normal((21, 8))
    o = _attend(rng.standard_normal(8), K, V)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-14)


def test_closed_form_dominant_key():
    rng = np.random.default_rng(2)
    K = np.zeros((30, 8))
    K[13, 0] = 40.0 / 0.25          # logit lead of 40 for q = e_0
    V = rng.standard_normal((30, 8))
    q = np.zeros(8)
    q[0] = 1.0
    o = _attend(q, K, V)
    np.testing.assert_allclose(o, V[13], atol=1e-15 * 30 + 30 * math.exp(-40) * 5)


# ------------------------------------------------------------------ invariants

def test_placement_permutation_invariance():
    w1 = workloads.make("llama7b_decode", num_seqs=6)
    w2 = workloads.make("llama7b_decode", num_seqs=6, placement="identity")
    assert not np.array_equal(w1.block_tables, w2.block_tables)
    o1 = run_oracle(w1)
    o2 = run_oracle(w2)
    assert np.array_equal(o1, o2)


def test_shared_prefix_equals_private_copies():
    ws = workloads.make("fp8_shared_prefix", num_seqs=3, prefix=256)
    wp = workloads.make("fp8_shared_prefix", num_seqs=3, prefix=256, placement="private")
    assert np.unique(ws.block_tables[:, :16]).size == 16         # prefix blocks are shared
    assert np.unique(wp.block_tables[:, :16]).size == 48         # ...or copied
    assert np.array_equal(run_oracle(ws), run_oracle(wp))


def test_block_size_invariance():
    outs = [run_oracle(workloads.make("fp8_shared_prefix", num_seqs=2, prefix=192, block_size=B))
            for B in (16, 32, 64)]
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(outs[0], outs[2], rtol=0, atol=1e-12)


def test_chunked_prefill_rows_equal_whole_prompt_rows():
    # one prompt of 96 tokens processed whole, vs. as its second chunk of 40 at offset 56
    whole = build("w", 21, [96], [96], num_q_heads=4, num_kv_heads=2, head_dim=32,
                  block_size=16, kv_dtype="bf16")
    chunk = build("c", 21, [96], [40], num_q_heads=4, num_kv_heads=2, head_dim=32,
                  block_size=16, kv_dtype="bf16")
    # same seed -> same K/V values; the chunk's queries are the whole prompt's last 40 rows
    qw = whole.q_values()
    kp, vp = C.fill_pools(whole)
    ow = A.paged_attention(qw, "bf16", kp, vp, "bf16", whole.block_tables, whole.seq_lens,
                           whole.query_start_loc, 16, whole.scale)
    kp2, vp2 = C.fill_pools(chunk)
    oc = A.paged_attention(qw[56:], "bf16", kp2, vp2, "bf16", chunk.block_tables, chunk.seq_lens,
                           chunk.query_start_loc, 16, chunk.scale)
    np.testing.assert_allclose(ow[56:], oc, rtol=0, atol=1e-12)
    # a decode row of length L equals the last row of a chunk ending at L
    dec = build("d", 21, [96], [1], num_q_heads=4, num_kv_heads=2, head_dim=32,
                block_size=16, kv_dtype="bf16")
    kp3, vp3 = C.fill_pools(dec)
    od = A.paged_attention(qw[95:], "bf16", kp3, vp3, "bf16", dec.block_tables, dec.seq_lens,
                           dec.query_start_loc, 16, dec.scale)
    np.testing.assert_allclose(ow[95:], od, rtol=0, atol=1e-12)


def test_lse_merge_of_partitions_reproduces_softmax():
    # split the keys of one row into partitions, keep (m, l, acc) per partition,
    # merge with weights exp(m_p - M): the result is the full softmax
    rng = np.random.default_rng(4)
    K, V, q = rng.standard_normal((300, 16)), rng.standard_normal((300, 16)), rng.standard_normal(16)
    full = _attend(q, K, V)
    for P in (1, 7, 64, 256, 300):
        ms, ls, accs = [], [], []
        for s0 in range(0, 300, P):
            s = 0.25 * K[s0:s0 + P] @ q
            m = s.max()
            w = np.exp(s - m)
            ms.append(m), ls.append(w.sum()), accs.append(w @ V[s0:s0 + P])
        M = max(ms)
        num = sum(math.exp(m - M) * a for m, a in zip(ms, accs))
        den = sum(math.exp(m - M) * l for m, l in zip(ms, ls))
        np.testing.assert_allclose(num / den, full, atol=1e-13)


def test_metadata_validation_rejects_bad_inputs():
    w = small_mixed()
    bt = w.block_tables.copy()
    bt[0, 0] = w.num_blocks
    with pytest.raises(ValueError):
        A.validate_metadata(w.seq_lens, w.query_start_loc, bt, w.num_blocks, w.block_size)
    qsl = w.query_start_loc.copy()
    qsl[1] = qsl[2] + 1
    with pytest.raises(ValueError):
        A.validate_metadata(w.seq_lens, qsl, w.block_tables, w.num_blocks, w.block_size)


def test_poisoned_tails_never_leak():
    # the pools hold NaN in every unwritten slot, yet the outputs are finite
    w = small_mixed("bf16")
    kp, vp = C.fill_pools(w)
    assert np.isnan(codecs.decode(kp, "bf16")).any()
    assert not np.isnan(run_oracle(w)).any()


# ------------------------------------------------------------------ cache write

@pytest.mark.parametrize("src,kv", [("f32", "f32"), ("bf16", "bf16"), ("f16", "f16"),
                                    ("f32", "bf16"), ("f32", "f16"), ("bf16", "fp8_e4m3"),
                                    ("f32", "fp8_e4m3"), ("f16", "fp8_e4m3")])
def test_cache_write_layout_and_roundtrip(src, kv):
    w = build("cw", 31, [37, 5, 16], [37, 5, 16], num_q_heads=2, num_kv_heads=2, head_dim=16,
              block_size=16, kv_dtype=kv, src_dtype=src, q_dtype="f32",
              k_scale=0.37 if kv == "fp8_e4m3" else 1.0, v_scale=0.11 if kv == "fp8_e4m3" else 1.0)
    kp, vp = C.fill_pools(w)
    poison = w.poison()
    written_k = np.zeros(kp.shape[:3], dtype=bool)    # [N][H][B]
    for i in range(w.num_seqs):
        k, v = w.kv_values(i)
        kf, vf = codecs.to_f32(k, src), codecs.to_f32(v, src)
        for pos, slot in enumerate(w.slots(i)):
            blk, off = int(slot) // 16, int(slot) % 16
            got_k = codecs.decode(kp[blk, :, off, :], kv) * w.k_scale
            got_v = codecs.decode(vp[blk, :, off, :], kv) * w.v_scale
            written_k[blk, :, off] = True
            if kv in ("f32",) or kv == src:
                assert np.array_equal(got_k, kf[pos].astype(np.float64))
                assert np.array_equal(got_v, vf[pos].astype(np.float64))
            elif kv == "fp8_e4m3":
                # within half an E4M3 quantum of the scaled value (relative 2^-4, absolute 2^-10)
                for got, ref, sc in ((got_k, kf[pos], w.k_scale), (got_v, vf[pos], w.v_scale)):
                    y = ref.astype(np.float64) / sc
                    err = np.abs(got / sc - y)
                    assert np.all(err <= np.maximum(np.abs(y) * 2 ** -4, 2 ** -10) + 1e-12)
            else:
                rel = 2 ** -8 if kv == "bf16" else 2 ** -11
                assert np.all(np.abs(got_k - kf[pos]) <= np.abs(kf[pos]) * rel + 6e-8)
    assert np.all(kp[~written_k] == poison) and np.all(vp[~written_k] == poison)
    assert written_k.sum() == w.num_kv_heads * int(w.seq_lens.sum())


def test_cache_write_skips_negative_slots():
    w = build("neg", 3, [8], [8], num_q_heads=1, num_kv_heads=1, head_dim=16, block_size=16,
              kv_dtype="bf16")
    kp, vp = w.initial_pool()
    k, v = w.kv_values(0)
    slots = w.slots(0).copy()
    slots[::2] = -1
    C.reshape_and_cache(kp, vp, k, v, "bf16", "bf16", slots, 16)
    blk = int(w.block_tables[0, 0])
    assert np.all(kp[blk, 0, 0::2, :] == w.poison())
    assert np.array_equal(kp[blk, 0, 1:8:2, :], k[1::2, 0, :])
    assert np.all(vp[blk, 0, 0::2, :] == w.poison())
    assert np.array_equal(vp[blk, 0, 1:8:2, :], v[1::2, 0, :])


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_same_format_write_equals_generic_rounding(dt):
    # the same-format shortcut must agree with widening to fp32 and rounding back
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 1 << 16, size=200_000, dtype=np.uint32).astype(np.uint16)
    src = bits if dt == "bf16" else bits.view(np.float16)
    short = C.encode_tokens(src, dt, dt, 1.0)
    generic = codecs.encode(codecs.to_f32(src, dt), dt)
    assert np.array_equal(short, generic)
