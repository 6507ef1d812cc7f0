"""Algorithmic work of a paged-attention step (bytes and FLOPs).

These are the figures a roofline is priced on: the bytes and FLOPs the
method itself must move and compute, independent of how a kernel tiles them.

* KV bytes: every cached K and V element a sequence attends is read once per
  (sequence, kv head): sum_i L_i * Hkv * 2 * d * eb.  The per-token factor is
  the same product the vLLM article (itwiki, "Background": OPT-13B example)
  uses for the size of a token's cache: 2 (K and V) x hidden x layers x bytes.
* FLOPs: 4 * d * Hq per visible (query, key) pair (2 for q.k, 2 for p.v).
  A decode row of length L sees L keys; a chunk of c tokens at offset o sees
  c*o + c*(c+1)/2 pairs under the causal mask.
"""

from __future__ import annotations

import numpy as np

from .generate import DTYPE_BYTES, Workload


def kv_bytes_per_token_model(hidden: int, layers: int, elem_bytes: int) -> int:
    """Cache bytes one token costs in a whole model: 2 x hidden x layers x eb."""
    return 2 * hidden * layers * elem_bytes


def workload_kv_bytes(w: Workload, unique: bool = False) -> int:
    """KV bytes one attention pass must read.

    unique=True counts each physical block once (a prefix whose blocks the
    tables share is then counted once instead of once per sequence; private
    copies of it count per sequence).
    """
    eb = DTYPE_BYTES[w.kv_dtype]
    per_token = w.num_kv_heads * 2 * w.head_dim * eb
    if not unique or not w.prefix_blocks_shared:
        return int(w.seq_lens.astype(np.int64).sum()) * per_token
    P = w.shared_prefix_len
    return (P + int((w.seq_lens.astype(np.int64) - P).sum())) * per_token


def workload_pairs(w: Workload) -> int:
    """Visible (query, key) pairs per q head under the causal mask."""
    L = w.seq_lens.astype(np.int64)
    c = w.query_lens.astype(np.int64)
    o = L - c
    return int((c * o + c * (c + 1) // 2).sum())


def workload_flops(w: Workload) -> int:
    return 4 * w.head_dim * w.num_q_heads * workload_pairs(w)


def step_other_bytes(w: Workload, with_cache_write: bool = True) -> int:
    """Bytes besides the KV cache: q, out, block tables, metadata, cache write."""
    ebq = DTYPE_BYTES[w.q_dtype]
    T = w.num_tokens
    b = T * w.num_q_heads * w.head_dim * 2 * ebq
    b += sum(w.blocks_of(i) for i in range(w.num_seqs)) * 4
    b += 4 * (2 * w.num_seqs + 1)
    if with_cache_write:
        b += T * w.num_kv_heads * 2 * w.head_dim * (DTYPE_BYTES[w.src_dtype] + DTYPE_BYTES[w.kv_dtype])
        b += T * 8
    return int(b)


def fragmentation(w: Workload) -> float:
    """Fraction of allocated slots left empty: only last blocks have holes."""
    L = w.seq_lens.astype(np.int64)
    alloc = (-(-L // w.block_size)) * w.block_size
    return float((alloc - L).sum() / max(1, alloc.sum()))
