"""The oracle over whole workloads at their full sizes, and the comparison
that reports each row's error beside its output's rounding step.

Requests are independent, and every request's cache tokens sit in slots of
their own, so the pool writes and the per-request attention of the oracle
are spread over a thread pool here; the oracle's arithmetic is unchanged
(``oracle.cache.reshape_and_cache`` and ``oracle.attention.attend_sequence``
do all of it).  Imported by the GPU parity tests only.
"""

from __future__ import annotations

import os
import sys
from collections import deque
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from oracle import codecs

TOL = {"f32": 2e-3, "f16": 2e-3, "bf16": 1e-2, "fp8_e4m3": 4e-2}
# bits kept after the leading one, by output dtype
_MANT = {"f32": 23, "f16": 10, "bf16": 7}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def fill_pools(w, seqs=None):
    """The pre-call pools with every cache token of ``seqs`` (all by default)
    written by the oracle's cache write (``oracle.cache.fill_pools``, with the
    writes of different requests -- disjoint slots -- run side by side)."""
    kp, vp = w.initial_pool()

    def put(x):
        _kind, _i, k, v, s = x
        oracle.cache.reshape_and_cache(kp, vp, k, v, w.src_dtype, w.kv_dtype, s, w.block_size,
                                       w.k_scale, w.v_scale)

    n = workers()
    with ThreadPoolExecutor(n) as ex:
        pending = deque()
        for x in w.iter_token_writes(seqs):
            pending.append(ex.submit(put, x))
            while len(pending) > 2 * n:
                pending.popleft().result()
        while pending:
            pending.popleft().result()
    return kp, vp


def attention(w, kp, vp, seqs=None):
    """``[T][Hq][d]`` float64 oracle output; rows of requests not in ``seqs`` are NaN."""
    from threadpoolctl import threadpool_limits

    oracle.attention.validate_metadata(w.seq_lens, w.query_start_loc, w.block_tables, w.num_blocks,
                                       w.block_size)
    qf = codecs.decode(w.q_values(), w.q_dtype)
    out = np.full(qf.shape, np.nan, dtype=np.float64)
    qsl = w.query_start_loc

    def one(i):
        a, b = int(qsl[i]), int(qsl[i + 1])
        if b > a:
            out[a:b] = oracle.attention.attend_sequence(qf[a:b], kp, vp, w.kv_dtype, w.block_tables[i],
                                                        int(w.seq_lens[i]), w.block_size, w.scale,
                                                        w.k_scale, w.v_scale)

    order = range(w.num_seqs) if seqs is None else seqs
    # longest requests first, so that the pool does not end on one of them
    order = sorted(order, key=lambda i: -int(w.seq_lens[i]) * int(w.query_lens[i]))
    with threadpool_limits(1), ThreadPoolExecutor(workers()) as ex:
        list(ex.map(one, order))
    return out


def rows_of(w, seqs):
    qsl = w.query_start_loc
    return np.concatenate([np.arange(qsl[i], qsl[i + 1]) for i in seqs]) if len(seqs) else \
        np.zeros(0, dtype=np.int64)


def half_ulp(x, dtype):
    """Half the spacing of ``dtype`` values at |x| (the rounding step of an
    output rounded to nearest)."""
    a = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(a)) - _MANT[dtype] - 1)


def assert_close(w, got, ref, seqs=None, label=""):
    """Every row of ``seqs`` (all by default): max-abs error within the
    tolerance of the cache dtype, no NaN.  Prints the worst row's error beside
    the half-ulp of that row's largest output, and the largest ratio of a
    row's error to its half-ulp (a diagnostic; the tolerance decides)."""
    rows = rows_of(w, range(w.num_seqs) if seqs is None else seqs)
    g, r = got[rows], ref[rows]
    assert not np.isnan(r).any(), f"{label}: the oracle left rows uncovered"
    assert not np.isnan(g).any(), f"{label}: NaN in GPU output"
    tol = TOL[w.kv_dtype]
    if g.size == 0:
        say(f"{label}: no rows")
        return
    err = np.abs(g - r).max(axis=-1)                     # per (token, q head)
    hu = half_ulp(np.abs(r).max(axis=-1), w.q_dtype)
    t, h = np.unravel_index(int(np.argmax(err)), err.shape)
    ratio = err / hu
    say(f"{label}: max-abs err {err.max():.3e} (tol {tol:.0e}) over {g.size} values, {err.size} rows; "
        f"worst row token {int(rows[t])} head {h}: |o|max {np.abs(r[t, h]).max():.3f}, half-ulp {hu[t, h]:.2e}; "
        f"largest err/half-ulp {ratio.max():.2f}")
    assert err.max() <= tol, f"{label}: max-abs error {err.max()} > {tol}"
