"""Cache write through a slot mapping (oracle side).

Each new token's K and V are written into the slot its request's block table
gives it: the vLLM 0.25 Model Runner V2 article (llm-wiki, "Redesign 3" and
"Redesign 4") names the slot mapping as the per-token input that says where a
token's cache entry goes; the itwiki "vLLM" article ("Block table") says a
request's cache is a run of fixed-size blocks and a new block is taken only
when the last one fills.

Reading of the slot encoding (the pages give none): slot = physical_block * B
+ offset_in_block, int64; a negative slot means "skip this token".

Pool layouts (the pages are silent on layout; this is the layout the library
defines): K and V are both ``[N][Hkv][B][d]``, i.e. each (block, head) tile
is contiguous and a token's d elements are one row of it.
"""

from __future__ import annotations

import numpy as np

from . import codecs


def encode_tokens(src: np.ndarray, src_dtype: str, kv_dtype: str, scale: float) -> np.ndarray:
    """Source K or V ``[T][Hkv][d]`` -> storage bits of the cache dtype.

    The source is widened to float32 exactly, then encoded: identity for an
    fp32 cache, RNE for fp16/bf16, and ``e4m3(fl32(x / scale))`` for fp8.
    """
    if src_dtype == kv_dtype and kv_dtype in ("bf16", "f16"):
        # a value already in the cache format rounds to itself; only NaN
        # payloads change, to the canonical quiet NaN with the sign kept
        bits = np.asarray(src)
        bits = bits.view(np.uint16) if bits.dtype != np.uint16 else bits
        mag = bits & np.uint16(0x7FFF)
        inf, qnan = (0x7F80, 0x7FC0) if kv_dtype == "bf16" else (0x7C00, 0x7E00)
        return np.where(mag > inf, (bits & np.uint16(0x8000)) | np.uint16(qnan), bits).astype(np.uint16)
    x = codecs.to_f32(src, src_dtype)
    return codecs.encode(x, kv_dtype, scale)


def reshape_and_cache(k_pool: np.ndarray, v_pool: np.ndarray, key: np.ndarray, value: np.ndarray,
                      src_dtype: str, kv_dtype: str, slot_mapping: np.ndarray, block_size: int,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Write every token with a non-negative slot into the pools, in place."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    if not np.any(keep):
        return
    s = slots[keep]
    blk = s // block_size
    off = s % block_size
    kb = encode_tokens(np.asarray(key)[keep], src_dtype, kv_dtype, k_scale)
    vb = encode_tokens(np.asarray(value)[keep], src_dtype, kv_dtype, v_scale)
    st = k_pool.dtype
    # K[blk][h][off][:] = enc(key[t][h][:]);  V[blk][h][off][:] = enc(value[t][h][:])
    k_pool[blk, :, off, :] = kb.astype(st, copy=False)
    v_pool[blk, :, off, :] = vb.astype(st, copy=False)


def fill_pools(workload, seqs=None):
    """Pre-call poisoned pools with every cache token of ``seqs`` written.

    Follows the workload's own write order: prior context first, then the
    step's new tokens, all through :func:`reshape_and_cache`.
    """
    kp, vp = workload.initial_pool()
    for _kind, _i, k, v, s in workload.iter_token_writes(seqs):
        reshape_and_cache(kp, vp, k, v, workload.src_dtype, workload.kv_dtype, s,
                          workload.block_size, workload.k_scale, workload.v_scale)
    return kp, vp
