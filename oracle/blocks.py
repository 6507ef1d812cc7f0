"""Whole-block copies between pools (oracle side) -- test infrastructure.

The itwiki "vLLM" article gives both uses.  Its section on block sharing
and copy-on-write: every physical block carries a reference count, and a
block that several sequences share is copied only when one of them must
write a new token into it.  Its section on scheduling and preemption: the
blocks of a preempted request leave together, to CPU memory from which they
are brought back later (swapping), or they are dropped and recomputed.

One operation covers both: block ``t`` of a destination pool becomes a copy
of block ``s`` of a source pool, for K and V, every kv head, bit for bit.
Pools are the raw storage bits in the layouts of ``oracle.cache``.

Readings (the pages give no interface): the mapping is a list of
``(src, dst)`` block pairs; a pair with an id outside its pool is skipped;
destinations must be distinct, and within one pool no destination may be a
source (otherwise the result would depend on the order of the copies).
"""

from __future__ import annotations

import numpy as np


def check_mapping(mapping: np.ndarray, src_blocks: int, dst_blocks: int, same_pool: bool) -> np.ndarray:
    """The pairs that take effect (ids inside their pools); raises ValueError
    when destinations repeat or, within one pool, a destination is a source."""
    m = np.asarray(mapping, dtype=np.int64).reshape(-1, 2)
    ok = (m[:, 0] >= 0) & (m[:, 0] < src_blocks) & (m[:, 1] >= 0) & (m[:, 1] < dst_blocks)
    m = m[ok]
    if len(np.unique(m[:, 1])) != len(m):
        raise ValueError("destination blocks repeat")
    if same_pool and np.intersect1d(m[:, 0], m[:, 1]).size:
        raise ValueError("a destination block is also a source within one pool")
    return m


def copy_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                mapping: np.ndarray) -> tuple:
    """Return new (K, V) destination pools: dst with block t replaced by src
    block s for every effective pair (s, t).  Inputs are not modified."""
    same = src_k is dst_k and src_v is dst_v
    m = check_mapping(mapping, src_k.shape[0], dst_k.shape[0], same)
    out_k, out_v = dst_k.copy(), dst_v.copy()
    for s, t in m:
        out_k[t] = src_k[s]
        out_v[t] = src_v[s]
    return out_k, out_v
