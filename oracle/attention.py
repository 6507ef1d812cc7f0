"""Paged attention, plain and slow, in float64 (oracle side).

The itwiki "vLLM" article, section "PagedAttention" > "Block-wise attention",
rewrites the attention of query i as a sum over B-token blocks K_j, V_j that
the kernel fetches one by one through the block table, and states that the
result is mathematically ordinary attention -- only the memory layout
changes.  So the oracle is ordinary attention, written out:

1. gather each request's blocks through its block table into contiguous
   K_i, V_i of L_i tokens (``gather_sequence``);
2. place the step's q_len_i queries at the last q_len_i positions,
   L_i - q_len_i + t (the chunked-prefill step of the vLLM V1 article,
   "Dynamic Chunked Prefill", mixes one-token decode rows with prompt chunks;
   query_start_loc, the cumulative per-request token counts, delimits them --
   llm-wiki MRV2 article, "Redesign 4");
3. for each query row and q head h (kv head h // (Hq/Hkv)): scores
   scale * K q over the keys at positions <= the query's, softmax with the
   maximum subtracted, weighted sum of V.

``block_sum_attention`` is the page's block-wise formula coded as printed
(per-block numerators, one normaliser summed over blocks, no maximum
subtraction), read straight from the pool; a test requires it to agree with
the gathered form.

Readings (the page's formula is garbled by extraction):
* the ones-vector in the normaliser sums a block's entries *outside* exp, so
  the denominator is the ordinary softmax normaliser;
* the causal limit is per token, not per block: a query sees keys at
  positions <= its own, never the later tokens of its last block;
* grouped-query heads map consecutively: q head h reads kv head h // G.
"""

from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from . import codecs


def validate_metadata(seq_lens, query_start_loc, block_tables, num_blocks, block_size):
    """The metadata invariants the path assumes; raises ValueError if broken."""
    seq_lens = np.asarray(seq_lens)
    qsl = np.asarray(query_start_loc)
    S = seq_lens.shape[0]
    if qsl.shape[0] != S + 1 or qsl[0] != 0:
        raise ValueError("query_start_loc must have S+1 entries starting at 0")
    qlen = np.diff(qsl)
    if np.any(qlen < 0):
        raise ValueError("query_start_loc must be non-decreasing")
    if np.any(qlen > seq_lens):
        raise ValueError("a sequence has more queries than cache tokens")
    nblk = -(-seq_lens.astype(np.int64) // block_size)
    if S and np.any(nblk > block_tables.shape[1]):
        raise ValueError("block table too narrow for a sequence")
    for i in range(S):
        ids = block_tables[i, :nblk[i]]
        if np.any(ids < 0) or np.any(ids >= num_blocks):
            raise ValueError(f"sequence {i} has a block id outside the pool")


def gather_sequence(k_pool, v_pool, kv_dtype, k_scale, v_scale, table_row, L, block_size):
    """Contiguous K, V ``[L][Hkv][d]`` in float64 for one request.

    Block j of the request is physical block ``table_row[j]``; K and V tiles
    are both ``[Hkv][B][d]`` in the pools.
    """
    nb = -(-int(L) // block_size)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    kt = k_pool[ids]                                   # [nb][Hkv][B][d]
    vt = v_pool[ids]                                   # [nb][Hkv][B][d]
    H, d = kt.shape[1], kt.shape[3]
    K = kt.transpose(0, 2, 1, 3).reshape(nb * block_size, H, d)[:L]
    V = vt.transpose(0, 2, 1, 3).reshape(nb * block_size, H, d)[:L]
    K = codecs.decode(K, kv_dtype) * float(k_scale)
    V = codecs.decode(V, kv_dtype) * float(v_scale)
    return K, V


def attend_rows(q, K, V, positions, scale, row_block: int = 128):
    """Ordinary causal attention of query rows over contiguous K/V.

    q ``[n][Hq][d]``; K, V ``[L][Hkv][d]``; positions ``[n]`` absolute
    positions of the rows.  Returns ``[n][Hq][d]`` float64.
    """
    n, Hq, d = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.empty((n, Hq, d), dtype=np.float64)
    Kt = np.ascontiguousarray(K.transpose(1, 0, 2))      # [Hkv][L][d]
    Vt = np.ascontiguousarray(V.transpose(1, 0, 2))      # [Hkv][L][d]
    keypos = np.arange(L)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        pos = np.asarray(positions[r0:r1])
        hi = int(pos.max()) + 1                          # keys any row here may see
        qb = q[r0:r1].reshape(r1 - r0, Hkv, G, d).transpose(1, 0, 2, 3)   # [Hkv][r][G][d]
        qb = qb.reshape(Hkv, (r1 - r0) * G, d)
        s = scale * (qb @ Kt[:, :hi, :].transpose(0, 2, 1))             # [Hkv][r*G][hi]
        s = s.reshape(Hkv, r1 - r0, G, hi)
        visible = keypos[None, :hi] <= pos[:, None]                       # [r][hi]
        s = np.where(visible[None, :, None, :], s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        w = np.exp(s - m)
        o = (w.reshape(Hkv, (r1 - r0) * G, hi) @ Vt[:, :hi, :]).reshape(Hkv, r1 - r0, G, d)
        o = o / w.sum(axis=-1)[..., None]
        out[r0:r1] = o.transpose(1, 0, 2, 3).reshape(r1 - r0, Hq, d)
    return out


def paged_attention(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, seq_lens, query_start_loc,
                    block_size, scale, k_scale=1.0, v_scale=1.0,
                    seqs: Optional[Iterable[int]] = None, validate: bool = True):
    """Output ``[T][Hq][d]`` float64 of one mixed step.

    q holds the storage representation of ``q_dtype`` (float32 values or
    16-bit patterns).  Rows of sequences not in ``seqs`` are NaN.
    """
    seq_lens = np.asarray(seq_lens)
    qsl = np.asarray(query_start_loc)
    if validate:
        validate_metadata(seq_lens, qsl, np.asarray(block_tables), k_pool.shape[0], block_size)
    qf = codecs.decode(q, q_dtype)
    out = np.full(qf.shape, np.nan, dtype=np.float64)
    S = seq_lens.shape[0]
    for i in (range(S) if seqs is None else seqs):
        a, b = int(qsl[i]), int(qsl[i + 1])
        if b > a:
            out[a:b] = attend_sequence(qf[a:b], k_pool, v_pool, kv_dtype, block_tables[i],
                                       int(seq_lens[i]), block_size, scale, k_scale, v_scale)
    return out


def attend_sequence(q_rows, k_pool, v_pool, kv_dtype, table_row, L, block_size, scale,
                    k_scale=1.0, v_scale=1.0):
    """Output ``[n][Hq][d]`` float64 of one request's n queries.

    q_rows ``[n][Hq][d]`` (decoded values) are the request's last n positions
    L - n .. L - 1; its L cached tokens are gathered through ``table_row``.
    Requests are independent of one another.
    """
    n = q_rows.shape[0]
    K, V = gather_sequence(k_pool, v_pool, kv_dtype, k_scale, v_scale, table_row, L, block_size)
    positions = L - n + np.arange(n)
    return attend_rows(q_rows, K, V, positions, scale)


def block_sum_attention(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, seq_lens,
                        query_start_loc, block_size, scale, k_scale=1.0, v_scale=1.0, seqs=None):
    """The block-wise formula, term by term, straight from the pool.

    For query i at position p and blocks j = 1..ceil((p+1)/B):
        A_ij = exp(q_i . K_j * scale) / sum_t sum_{k in block t} exp(q_i . k * scale)
        o_i  = sum_j V_j A_ij^T
    with keys past p (and past the sequence end) left out of every sum.
    """
    seq_lens = np.asarray(seq_lens)
    qsl = np.asarray(query_start_loc)
    qf = codecs.decode(q, q_dtype)
    T, Hq, d = qf.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    B = block_size
    out = np.full(qf.shape, np.nan, dtype=np.float64)
    for i in (range(seq_lens.shape[0]) if seqs is None else seqs):
        a, b = int(qsl[i]), int(qsl[i + 1])
        L = int(seq_lens[i])
        for t in range(b - a):
            p = L - (b - a) + t
            nblocks = p // B + 1                       # ceil((p + 1) / B)
            numer = [None] * nblocks
            vblk = [None] * nblocks
            for j in range(nblocks):
                phys = int(block_tables[i][j])
                n_in = min(B, p + 1 - j * B)           # keys of block j at positions <= p
                Kj = codecs.decode(k_pool[phys][:, :n_in, :], kv_dtype) * k_scale   # [Hkv][n][d]
                Vj = codecs.decode(v_pool[phys][:, :n_in, :], kv_dtype) * v_scale   # [Hkv][n][d]
                qh = qf[a + t].reshape(Hkv, G, d)
                numer[j] = np.exp(scale * np.einsum("hgd,hkd->hgk", qh, Kj))       # [Hkv][G][n]
                vblk[j] = Vj
            denom = sum(nj.sum(axis=-1) for nj in numer)                        # [Hkv][G]
            o = np.zeros((Hkv, G, d))
            for j in range(nblocks):
                A = numer[j] / denom[..., None]
                # V_j A_ij^T, V_j being the block's values as d x n columns
                o += np.einsum("hkd,hgk->hgd", vblk[j], A)
            out[a + t] = o.reshape(Hq, d)
    return out
