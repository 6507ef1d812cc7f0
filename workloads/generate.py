"""Seeded synthetic paged-attention workloads.

Recipe (every draw comes from ``numpy.random.default_rng`` seeded with a list
``[seed, stream, ...]`` so that any one sequence can be regenerated alone):

* stream 0 -- sequence lengths (and suffix lengths for a shared prefix);
* stream 1 -- physical placement: a random permutation of the block pool,
  consumed in (sequence, logical block) order;
* stream [2, i] -- K then V values of sequence i, token-major ``[L_i][Hkv][d]``,
  N(0, 1) drawn in float32;
* stream 3 -- K then V values of a shared prefix (all sequences see the same
  prefix tokens and the same physical blocks);
* stream 4 -- the step's queries ``[T][Hq][d]``, N(0, 1) in float32.

Values are handed over in their storage dtype: float32 as drawn; float16 as
numpy's cast of the draw; bfloat16 as the upper 16 bits of the float32 draw
(a random bfloat16 value, not a rounding of anything).  Unused slots and
unused blocks of the pool hold a quiet-NaN pattern, so any kernel that reads
past a sequence's end is caught.

The pool is sized 1.2x the blocks the batch needs (the LLaMA-7B decode shape
states this ratio; the other shapes reuse it).  Padding entries of a block
table point at a spare, poisoned block, so they are valid indices that hold
no data.

The configurations follow the paged-attention workloads of the pages: decode
steps (one query token per sequence), a chunked-prefill step that mixes
decode tokens with prompt chunks under a 4,096-token budget, and a shared
8,000-token system prompt whose blocks every sequence's table points at.
"""

from __future__ import annotations

import inspect
import math
import os
from collections import deque
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Dict, Iterator, List, Optional, Sequence, Tuple

import numpy as np

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}

# Quiet-NaN bit patterns used to poison never-written cache memory.
_POISON = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F}
_STORAGE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8_e4m3": np.uint8}


def poison_pattern(dtype: str) -> int:
    """Bit pattern (an unsigned int of the dtype's width) of the poison value."""
    return _POISON[dtype]


def storage_type(dtype: str):
    """Unsigned numpy type with the dtype's width (raw-bits view)."""
    return _STORAGE[dtype]


def draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) values in the storage representation of ``dtype``.

    f32 -> np.float32, f16 -> np.float16, bf16 -> np.uint16 bit patterns.
    """
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        # the high half of each little-endian float32
        return np.ascontiguousarray(x.view(np.uint16)[..., 1::2])
    raise ValueError(f"no source representation for {dtype}")


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str          # cache storage: f32 | f16 | bf16 | fp8_e4m3
    src_dtype: str         # dtype of the K/V handed to the cache write
    q_dtype: str           # dtype of q and of the output
    k_scale: float
    v_scale: float
    seq_lens: np.ndarray           # int32 [S]: cache tokens incl. this step's
    query_lens: np.ndarray         # int32 [S]
    num_blocks: int                # physical pool size N
    block_tables: np.ndarray       # int32 [S][max_blocks_per_seq]
    spare_block: int               # an unused (poisoned) block id
    shared_prefix_len: int = 0     # tokens of a prefix common to every sequence
    prefix_blocks_shared: bool = True  # False: each sequence owns copies of them
    description: str = ""
    extra: Dict = field(default_factory=dict)

    # ---- derived shapes -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def query_start_loc(self) -> np.ndarray:
        qsl = np.zeros(self.num_seqs + 1, dtype=np.int32)
        np.cumsum(self.query_lens, out=qsl[1:])
        return qsl

    @property
    def num_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the float32 the kernel receives."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def blocks_of(self, i: int) -> int:
        return -(-int(self.seq_lens[i]) // self.block_size)

    # ---- values ---------------------------------------------------------
    def _prefix_values(self) -> Tuple[np.ndarray, np.ndarray]:
        cached = self.extra.get("_prefix")
        if cached is None:
            rng = np.random.default_rng([self.seed, 3])
            shape = (self.shared_prefix_len, self.num_kv_heads, self.head_dim)
            k = draw_values(rng, shape, self.src_dtype)
            v = draw_values(rng, shape, self.src_dtype)
            cached = (k, v)
            self.extra["_prefix"] = cached
        return cached

    def kv_values(self, i: int) -> Tuple[np.ndarray, np.ndarray]:
        """K and V of every cache position of sequence i, ``[L_i][Hkv][d]``."""
        L = int(self.seq_lens[i])
        rng = np.random.default_rng([self.seed, 2, i])
        own = L - self.shared_prefix_len
        shape = (own, self.num_kv_heads, self.head_dim)
        k = draw_values(rng, shape, self.src_dtype)
        v = draw_values(rng, shape, self.src_dtype)
        if self.shared_prefix_len:
            pk, pv = self._prefix_values()
            k = np.concatenate([pk, k], axis=0)
            v = np.concatenate([pv, v], axis=0)
        return k, v

    def iter_kv_values(self, seqs: Sequence[int], workers: Optional[int] = None,
                       lookahead: int = 16) -> Iterator[Tuple[np.ndarray, np.ndarray]]:
        """``kv_values(i)`` for each i in order, drawn on a small thread pool
        (every sequence has its own generator, so the values do not depend on
        the pool)."""
        if self.shared_prefix_len:
            self._prefix_values()
        workers = workers or min(16, os.cpu_count() or 1)
        if workers <= 1 or len(seqs) <= 1:
            for i in seqs:
                yield self.kv_values(i)
            return
        with ThreadPoolExecutor(workers) as ex:
            pending = deque()
            it = iter(seqs)
            for i in it:
                pending.append(ex.submit(self.kv_values, i))
                if len(pending) >= lookahead:
                    break
            for i in it:
                yield pending.popleft().result()
                pending.append(ex.submit(self.kv_values, i))
            while pending:
                yield pending.popleft().result()

    def q_values(self) -> np.ndarray:
        """Queries of the step, ``[T][Hq][d]`` in the q dtype."""
        rng = np.random.default_rng([self.seed, 4])
        return draw_values(rng, (self.num_tokens, self.num_q_heads, self.head_dim), self.q_dtype)

    def slots(self, i: int) -> np.ndarray:
        """Slot (physical block * B + offset) of each cache position of seq i."""
        L = int(self.seq_lens[i])
        pos = np.arange(L, dtype=np.int64)
        blocks = self.block_tables[i, pos // self.block_size].astype(np.int64)
        return blocks * self.block_size + pos % self.block_size

    # ---- cache writes ---------------------------------------------------
    def iter_token_writes(self, seqs: Optional[Sequence[int]] = None
                          ) -> Iterator[Tuple[str, int, np.ndarray, np.ndarray, np.ndarray]]:
        """Yield ``(kind, seq, key, value, slots)`` covering every cache token.

        kind is "prior" for context that was cached before this step and
        "new" for this step's tokens (the last ``q_len`` positions of each
        sequence, yielded in batch order).  A shared prefix is yielded once,
        as "prior", with seq = -1, when its blocks are shared; a prefix held in
        private copies is written with each sequence.
        """
        seqs = list(range(self.num_seqs)) if seqs is None else list(seqs)
        P = self.shared_prefix_len if self.prefix_blocks_shared else 0
        if P and len(seqs):
            pk, pv = self._prefix_values()
            yield "prior", -1, pk, pv, self.slots(seqs[0])[:P]
        for i, (k, v) in zip(seqs, self.iter_kv_values(seqs)):
            s = self.slots(i)
            L = int(self.seq_lens[i])
            n_new = int(self.query_lens[i])
            cut = L - n_new
            if cut > P:
                yield "prior", i, k[P:cut], v[P:cut], s[P:cut]
            if n_new:
                yield "new", i, k[cut:], v[cut:], s[cut:]

    def new_token_batch(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """This step's key/value ``[T][Hkv][d]`` and int64 slot mapping ``[T]``."""
        ks, vs, ss = [], [], []
        seqs = [i for i in range(self.num_seqs) if int(self.query_lens[i])]
        for i, (k, v) in zip(seqs, self.iter_kv_values(seqs)):
            n_new = int(self.query_lens[i])
            ks.append(k[-n_new:])
            vs.append(v[-n_new:])
            ss.append(self.slots(i)[-n_new:])
        shape = (0, self.num_kv_heads, self.head_dim)
        if not ks:
            e = np.zeros(shape, dtype=draw_values(np.random.default_rng(0), (0,), self.src_dtype).dtype)
            return e, e.copy(), np.zeros(0, dtype=np.int64)
        return np.concatenate(ks), np.concatenate(vs), np.concatenate(ss)

    def initial_pool(self) -> Tuple[np.ndarray, np.ndarray]:
        """Pre-call pool images (raw bits) filled with the poison pattern.

        K and V are both ``[N][Hkv][B][d]`` and hold the storage bits of
        ``kv_dtype``.
        """
        st = storage_type(self.kv_dtype)
        N, H, B, d = self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim
        k = np.full((N, H, B, d), self.poison(), dtype=st)
        v = np.full((N, H, B, d), self.poison(), dtype=st)
        return k, v

    def poison(self) -> int:
        return poison_pattern(self.kv_dtype)

    def summary(self) -> Dict:
        return dict(name=self.name, seqs=self.num_seqs, tokens=self.num_tokens,
                    q_heads=self.num_q_heads, kv_heads=self.num_kv_heads,
                    head_dim=self.head_dim, block_size=self.block_size,
                    kv_dtype=self.kv_dtype, q_dtype=self.q_dtype,
                    max_seq_len=self.max_seq_len, max_query_len=self.max_query_len,
                    num_blocks=self.num_blocks, shared_prefix=self.shared_prefix_len)


# ---------------------------------------------------------------------------
# builder
# ---------------------------------------------------------------------------

def build(name: str, seed: int, seq_lens: Sequence[int], query_lens: Sequence[int], *,
          num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
          kv_dtype: str, src_dtype: Optional[str] = None, q_dtype: Optional[str] = None,
          k_scale: float = 1.0, v_scale: float = 1.0, placement: str = "shuffled",
          pool_factor: float = 1.2, num_blocks: Optional[int] = None,
          shared_prefix_len: int = 0, description: str = "") -> Workload:
    """Assemble a workload from lengths; draws placement from stream 1.

    placement: "shuffled" (random physical ids), "identity" (contiguous ids in
    (sequence, block) order), or "private" (like shuffled, but a shared prefix
    is copied into every sequence's own blocks instead of being shared).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    assert seq_lens.shape == query_lens.shape
    assert np.all(query_lens <= seq_lens) and np.all(query_lens >= 0)
    if src_dtype is None:
        src_dtype = kv_dtype if kv_dtype != "fp8_e4m3" else "bf16"
    if q_dtype is None:
        q_dtype = src_dtype
    B = block_size
    S = len(seq_lens)
    nblk = [-(-int(L) // B) for L in seq_lens]
    share = shared_prefix_len if placement != "private" else 0
    if shared_prefix_len:
        assert shared_prefix_len % B == 0, "a shared prefix must fill whole blocks"
        assert np.all(seq_lens >= shared_prefix_len)
    nsh = share // B
    private = [n - nsh for n in nblk]
    needed = nsh + sum(private)
    if num_blocks is None:
        num_blocks = nsh + int(math.ceil(pool_factor * sum(private)))
        num_blocks = max(num_blocks, needed + 1)
    assert num_blocks >= needed + 1, "pool needs one spare block for table padding"
    rng = np.random.default_rng([seed, 1])
    if placement == "identity":
        ids = np.arange(num_blocks, dtype=np.int64)
    else:
        ids = rng.permutation(num_blocks)
    shared_ids = ids[:nsh]
    cursor = nsh
    max_blocks = max(nblk) if S else 1
    max_blocks = max(max_blocks, 1)
    spare = int(ids[needed])
    tables = np.full((S, max_blocks), spare, dtype=np.int32)
    for i in range(S):
        tables[i, :nsh] = shared_ids
        n = private[i]
        tables[i, nsh:nsh + n] = ids[cursor:cursor + n]
        cursor += n
    return Workload(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=B, kv_dtype=kv_dtype, src_dtype=src_dtype,
                    q_dtype=q_dtype, k_scale=float(k_scale), v_scale=float(v_scale),
                    seq_lens=seq_lens, query_lens=query_lens, num_blocks=int(num_blocks),
                    block_tables=tables, spare_block=spare,
                    shared_prefix_len=int(shared_prefix_len),
                    prefix_blocks_shared=bool(nsh > 0) or not shared_prefix_len,
                    description=description)


# ---------------------------------------------------------------------------
# the named configurations
# ---------------------------------------------------------------------------

FP8_SCALE = 2.0 ** -5   # power of two: x / scale is exact, N(0,1)/scale stays far below 448


def _tiny_decode(num_seqs=None, **kw) -> Workload:
    seed = 141001
    lens = [1, 7, 16, 33]
    return build("tiny_decode", seed, lens, [1] * 4, num_q_heads=2, num_kv_heads=2,
                 head_dim=64, block_size=16, kv_dtype=kw.pop("kv_dtype", "f32"),
                 num_blocks=16, description="4 decode seqs, lengths {1,7,16,33}, fp32", **kw)


def _llama7b_decode(num_seqs=256, placement="shuffled", block_size=16, **kw) -> Workload:
    seed = 141002
    rng = np.random.default_rng([seed, 0])
    lens = rng.integers(128, 2048, size=256, endpoint=True)[:num_seqs]
    name = "llama7b_decode" + ("_identity" if placement == "identity" else "")
    return build(name, seed, lens, [1] * len(lens), num_q_heads=32, num_kv_heads=32,
                 head_dim=128, block_size=block_size, kv_dtype=kw.pop("kv_dtype", "bf16"),
                 placement=placement,
                 description="LLaMA-7B-shaped decode: 32/32 heads, d=128, L~U[128,2048]", **kw)


def _gqa_long_decode(num_seqs=64, head_dim=128, block_size=16, **kw) -> Workload:
    """head_dim=256 keeps the KV bytes per token with 16q/4kv heads."""
    seed = 141003
    rng = np.random.default_rng([seed, 0])
    lens = np.floor(np.exp(rng.uniform(math.log(1024), math.log(32768), size=64))).astype(np.int64)
    lens = lens[:num_seqs]
    hq, hkv = (32, 8) if head_dim == 128 else (32 * 128 // head_dim, 8 * 128 // head_dim)
    return build("gqa_long_decode" + ("" if head_dim == 128 else f"_d{head_dim}"), seed, lens, [1] * len(lens),
                 num_q_heads=hq, num_kv_heads=hkv, head_dim=head_dim, block_size=block_size,
                 kv_dtype=kw.pop("kv_dtype", "bf16"),
                 description=f"GQA decode, {hq}q/{hkv}kv, d {head_dim}, L log-uniform in [1k, 32k]", **kw)


def _mixed_chunked_prefill(num_seqs=256, chunk_scale=1, head_dim=128, block_size=16, **kw) -> Workload:
    """256 decode tokens, then prompt chunks (offset, length) in batch order.

    chunk_scale divides the chunk lengths and offsets (for reduced copies).
    """
    seed = 141004
    rng = np.random.default_rng([seed, 0])
    dec = rng.integers(256, 4096, size=256, endpoint=True)[:num_seqs]
    chunks = [(0, 1024), (4096, 1024), (8192, 1024), (0, 512)]
    chunks = [(o // chunk_scale, c // chunk_scale) for o, c in chunks]
    lens = list(dec) + [o + c for o, c in chunks]
    qlens = [1] * len(dec) + [c for _, c in chunks]
    hq, hkv = (32, 8) if head_dim == 128 else (32 * 128 // head_dim, 8 * 128 // head_dim)
    return build("mixed_chunked_prefill" + ("" if head_dim == 128 else f"_d{head_dim}"), seed, lens, qlens,
                 num_q_heads=hq, num_kv_heads=hkv, head_dim=head_dim, block_size=block_size,
                 kv_dtype=kw.pop("kv_dtype", "bf16"),
                 description="256 decode tokens + chunks 3x1024 (offsets 0/4096/8192) + 512, "
                             "4096-token budget, 32q/8kv, d=128", **kw)


def _fp8_shared_prefix(num_seqs=128, block_size=16, placement="shuffled", prefix=8000, **kw) -> Workload:
    seed = 141005
    rng = np.random.default_rng([seed, 0])
    suffix = rng.integers(64, 512, size=128, endpoint=True)[:num_seqs]
    lens = prefix + suffix
    tag = "private" if placement == "private" else "shared"
    return build(f"fp8_{tag}_prefix_B{block_size}", seed, lens, [1] * len(lens), num_q_heads=32,
                 num_kv_heads=8, head_dim=128, block_size=block_size,
                 kv_dtype=kw.pop("kv_dtype", "fp8_e4m3"), src_dtype="bf16", q_dtype="bf16",
                 k_scale=FP8_SCALE, v_scale=FP8_SCALE, placement=placement,
                 shared_prefix_len=prefix,
                 description=f"fp8 KV, {prefix}-token shared prefix + private suffix U[64,512]",
                 **kw)


CONFIGS: Dict[str, Callable[..., Workload]] = {
    "tiny_decode": _tiny_decode,
    "llama7b_decode": _llama7b_decode,
    "gqa_long_decode": _gqa_long_decode,
    "mixed_chunked_prefill": _mixed_chunked_prefill,
    "fp8_shared_prefix": _fp8_shared_prefix,
}


def make(name: str, **kw) -> Workload:
    """Build a named configuration; keyword arguments shrink or vary it."""
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
    if "head_dim" in kw and "head_dim" not in inspect.signature(CONFIGS[name]).parameters:
        raise ValueError(f"{name} fixes its head dim; it takes no head_dim override")
    return CONFIGS[name](**kw)


def random_mixed(seed: int, *, num_decode: int, chunk_specs: Sequence[Tuple[int, int]],
                 max_decode_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, kv_dtype: str, q_dtype: Optional[str] = None,
                 src_dtype: Optional[str] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                 min_decode_len: int = 1, placement: str = "shuffled",
                 name: str = "random_mixed") -> Workload:
    """Small mixed batch for parity tests: decode rows with random lengths plus
    chunks given as (offset, length)."""
    rng = np.random.default_rng([seed, 0])
    dec = rng.integers(min_decode_len, max_decode_len, size=num_decode, endpoint=True)
    lens = list(dec) + [o + c for o, c in chunk_specs]
    qlens = [1] * num_decode + [c for _, c in chunk_specs]
    return build(name, seed, lens, qlens, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, block_size=block_size, kv_dtype=kv_dtype,
                 q_dtype=q_dtype, src_dtype=src_dtype, k_scale=k_scale, v_scale=v_scale,
                 placement=placement)
