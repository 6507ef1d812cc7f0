"""Pins for the whole-block copy oracle (CPU only).

Copy-on-write and swapping are pinned by what the itwiki "vLLM" article says
they are for, checked against pools built a different way:
* copy-on-write (section on block sharing): two sequences share a prompt
  whose last block is partly filled; the one that writes next gets a copy of
  that block first.  Both must then attend exactly as if each had written its
  tokens into blocks of its own from the start;
* swapping (section on scheduling and preemption): a request's blocks go out
  to a host pool and come back into other device blocks; with the block table
  updated, attention is unchanged;
plus the readings: out-of-range pairs are skipped, repeated destinations and
in-pool overlaps are refused, and no other block changes.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import blocks as BL
from oracle import cache as C
from oracle import codecs

B, H, D = 16, 2, 32
SCALE = 1.0 / np.sqrt(D)


def tokens(rng, n):
    k = rng.standard_normal((n, H, D)).astype(np.float32)
    v = rng.standard_normal((n, H, D)).astype(np.float32)
    return k, v


def empty_pool(n):
    nan = np.uint32(0x7FC00000)   # fp32 poison: a block nobody wrote
    return np.full((n, H, B, D), nan, np.uint32), np.full((n, H, B, D), nan, np.uint32)


def write(kp, vp, k, v, slots):
    C.reshape_and_cache(kp, vp, k, v, "f32", "f32", np.asarray(slots, np.int64), B)


def attend(kp, vp, q, tables, lens):
    tables = np.asarray(tables, np.int32)
    lens = np.asarray(lens, np.int32)
    qsl = np.arange(len(lens) + 1, dtype=np.int32)
    return A.paged_attention(q, "f32", kp, vp, "f32", tables, lens, qsl, B, SCALE)


def test_copy_on_write_equals_private_blocks():
    rng = np.random.default_rng(1)
    P = 40                                     # shared prompt: blocks 0, 1 full, block 2 holds 8 tokens
    kprompt, vprompt = tokens(rng, P)
    ka, va = tokens(rng, 1)                    # the next token of sequence a
    kb, vb = tokens(rng, 1)                    # ... and of sequence b
    q = rng.standard_normal((2, H, D)).astype(np.float32)

    # shared: both tables point at blocks 3, 7, 5; b copies block 5 to 9 before writing
    kp, vp = empty_pool(12)
    write(kp, vp, kprompt, vprompt, [[3, 7, 5][t // B] * B + t % B for t in range(P)])
    kp, vp = BL.copy_blocks(kp, vp, kp, vp, np.array([[5, 9]]))
    write(kp, vp, ka, va, [5 * B + 8])
    write(kp, vp, kb, vb, [9 * B + 8])
    shared = attend(kp, vp, q, [[3, 7, 5], [3, 7, 9]], [P + 1, P + 1])

    # private: each sequence wrote the prompt and its own token into blocks of its own
    kq, vq = empty_pool(12)
    write(kq, vq, kprompt, vprompt, [[0, 1, 2][t // B] * B + t % B for t in range(P)])
    write(kq, vq, kprompt, vprompt, [[4, 6, 8][t // B] * B + t % B for t in range(P)])
    write(kq, vq, ka, va, [2 * B + 8])
    write(kq, vq, kb, vb, [8 * B + 8])
    private = attend(kq, vq, q, [[0, 1, 2], [4, 6, 8]], [P + 1, P + 1])
    assert not np.isnan(shared).any()
    np.testing.assert_array_equal(shared, private)

    # without the copy, b's write would land in a's block: a would see b's token
    kn, vn = empty_pool(12)
    write(kn, vn, kprompt, vprompt, [[3, 7, 5][t // B] * B + t % B for t in range(P)])
    write(kn, vn, ka, va, [5 * B + 8])
    write(kn, vn, kb, vb, [5 * B + 8])
    no_cow = attend(kn, vn, q, [[3, 7, 5]], [P + 1])
    assert not np.array_equal(no_cow[0], private[0])


def test_swap_out_and_back_leaves_attention_unchanged():
    rng = np.random.default_rng(2)
    L = 57
    k, v = tokens(rng, L)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    kp, vp = empty_pool(10)
    table = [6, 1, 8, 3]
    write(kp, vp, k, v, [table[t // B] * B + t % B for t in range(L)])
    before = attend(kp, vp, q, [table], [L])
    hk, hv = empty_pool(5)                                       # the host pool
    hk, hv = BL.copy_blocks(kp, vp, hk, hv, np.array([[6, 4], [1, 0], [8, 2], [3, 1]]))
    kp2, vp2 = empty_pool(10)                                    # the device blocks were reused meanwhile
    kp2, vp2 = BL.copy_blocks(hk, hv, kp2, vp2, np.array([[4, 9], [0, 2], [2, 5], [1, 7]]))
    after = attend(kp2, vp2, q, [[9, 2, 5, 7]], [L])
    np.testing.assert_array_equal(before, after)


def test_only_destinations_change_and_out_of_range_pairs_are_skipped():
    rng = np.random.default_rng(3)
    kp = rng.integers(0, 2 ** 32, size=(8, H, B, D), dtype=np.uint32)
    vp = rng.integers(0, 2 ** 32, size=(8, H, B, D), dtype=np.uint32)
    m = np.array([[0, 5], [2, 6], [-1, 7], [3, 8], [9, 1]])     # the last three are out of range
    ok, ov = BL.copy_blocks(kp, vp, kp, vp, m)
    for t in range(8):
        src = {5: 0, 6: 2}.get(t, t)
        np.testing.assert_array_equal(ok[t], kp[src])
        np.testing.assert_array_equal(ov[t], vp[src])
    assert BL.check_mapping(m, 8, 8, True).tolist() == [[0, 5], [2, 6]]


def test_refuses_order_dependent_mappings():
    kp, vp = empty_pool(6)
    with pytest.raises(ValueError):
        BL.copy_blocks(kp, vp, kp, vp, np.array([[0, 3], [1, 3]]))    # destination repeats
    with pytest.raises(ValueError):
        BL.copy_blocks(kp, vp, kp, vp, np.array([[0, 3], [3, 4]]))    # a destination is a source
    hk, hv = empty_pool(6)
    BL.copy_blocks(kp, vp, hk, hv, np.array([[0, 3], [3, 4]]))        # fine between two pools


def test_fp8_blocks_copy_bytes():
    rng = np.random.default_rng(4)
    kp = rng.integers(0, 256, size=(4, H, B, D), dtype=np.uint8)
    vp = rng.integers(0, 256, size=(4, H, B, D), dtype=np.uint8)
    ok, ov = BL.copy_blocks(kp, vp, kp, vp, np.array([[1, 3]]))
    assert ok.dtype == np.uint8 and ok[3].tobytes() == kp[1].tobytes() and ov[3].tobytes() == vp[1].tobytes()
    assert codecs.decode(ok[3], "fp8_e4m3").shape == (H, B, D)
