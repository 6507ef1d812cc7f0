"""MI355X (gfx950) paged attention -- Python face of ``libpa.so``.

A thin ``ctypes`` binding over the C ABI in ``include/pa.h``: it checks
tensor shapes and dtypes, passes raw device pointers, sizes and the current
torch stream, and turns status codes into exceptions.  Every step of the
computation runs in the library's HIP kernels; torch only provides device
memory and the stream.  If the library is not built this module raises on
first use -- there is no other path.

    k_cache: [num_blocks, num_kv_heads, block_size, head_dim]
    v_cache: [num_blocks, num_kv_heads, head_dim, block_size]
    dtypes : torch.float32 / float16 / bfloat16, or torch.float8_e4m3fn
             (uint8 storage is accepted as fp8 codes).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "PagedAttentionError", "library", "library_path", "reshape_and_cache", "attention",
    "attention_workspace_size", "check_metadata", "copy_blocks", "apply_block_table_writes", "prepare_step", "commit_step",
    "set_attention_events", "preferred_block_size", "attention_noalloc", "NOALLOC_SCRATCH_BYTES", "PA_F32", "PA_F16",
    "PA_BF16", "PA_FP8_E4M3",
]

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_OK = 0
PA_ERR_METADATA = 7
PA_ERR_TOO_LARGE = 8
NOALLOC_SCRATCH_BYTES = 64 << 20      # PA_NOALLOC_SCRATCH_BYTES of include/pa.h

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "_lib", "libpa.so")
debug_library_path = os.path.join(_HERE, "_lib", "libpa_debug.so")


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class _Cache(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


_lib = None


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m paged_kv_cache_141_amd.build`")
    try:
        # torch ships its own HIP runtime with the same soname; loading torch
        # first makes the library bind to that one runtime (one set of streams)
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    CP = ctypes.POINTER(_Cache)
    sig = {
        "pa_reshape_and_cache": [P, P, I32, P, P, CP, P, I32, P],
        "pa_attention_workspace_size": [CP, I32, I32, I32, I32, I32, ctypes.POINTER(SZ)],
        "pa_attention": [P, I32, P, P, CP, P, I32, P, P, I32, I32, I32, I32, I32, F, P, P, SZ, P],
        "pa_write_and_attend": [P, P, I32, P, I32, P, I32, P, P, CP, P, I32, P, P, I32, I32, I32, I32, I32, I32, F,
                                P, P, SZ, P],
        "pa_attention_noalloc": [P, I32, P, P, CP, P, I32, P, P, I32, I32, I32, I32, I32, F, P, P],
        "pa_preferred_block_size": [I32, I32, I32, I32, ctypes.POINTER(I32)],
        "pa_attention_shared_prefix_workspace_size": [CP, I32, I32, I32, I32, I32, I32, ctypes.POINTER(SZ)],
        "pa_attention_shared_prefix": [P, I32, P, P, CP, P, I32, P, P, I32, I32, I32, I32, I32, I32, F, P, P, SZ, P],
        "pa_check_metadata": [CP, P, I32, P, P, I32, I32, I32, I32, ctypes.POINTER(I32), P],
        "pa_debug_check": [ctypes.POINTER(I32), ctypes.POINTER(I32), P],
        "pa_copy_blocks": [P, P, CP, P, P, CP, P, I32, P],
        "pa_apply_block_table_writes": [P, I32, I32, P, P, P, P, I32, I32, P],
        "pa_prepare_step": [P, I32, I32, P, P, P, I32, I32, I32, P, P, P, P, P, P],
        "pa_commit_step": [P, I32, P, P, I32, P],
        "pa_set_attention_events": [P, P],
        "pa_set_chunk_events": [P, P],
        "pa_set_prefix_events": [P, P],
        "pa_status_string": [I32],
        "pa_version": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("pa_status_string", "pa_version") else ctypes.c_int
    return lib


def library() -> ctypes.CDLL:
    """Load ``libpa.so`` (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        _lib = _load(library_path)
    return _lib


_debug_lib = None


def debug_library() -> ctypes.CDLL:
    """Load ``libpa_debug.so``, the library built with -DPA_DEBUG=1 (the same
    entry points, with metadata, block-id and slot checks recorded for
    ``pa_debug_check``); raise if it is missing."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(debug_library_path)
    return _debug_lib


def debug_check(lib=None, stream=None):
    """``pa_debug_check`` of the debug library: (code, index) of the first
    recorded violation, (0, 0) if none; the record is cleared."""
    lib = lib or debug_library()
    code, index = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.pa_debug_check(ctypes.byref(code), ctypes.byref(index), _stream(stream))
    if st not in (PA_OK, PA_ERR_METADATA):
        raise PagedAttentionError(st, "pa_debug_check")
    return int(code.value), int(index.value)


def status_string(status: int) -> str:
    return library().pa_status_string(status).decode()


def version() -> str:
    return library().pa_version().decode()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
         torch.uint8: PA_FP8_E4M3}
    if hasattr(torch, "float8_e4m3fn"):
        m[torch.float8_e4m3fn] = PA_FP8_E4M3
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def cache_spec(k_cache, v_cache, k_scale: float = 1.0, v_scale: float = 1.0) -> _Cache:
    if k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("caches must be 4-D")
    N, H, B, d = k_cache.shape
    if tuple(v_cache.shape) != (N, H, B, d):
        raise ValueError(f"v_cache must be [N, Hkv, B, d] = {(N, H, B, d)}, got {tuple(v_cache.shape)}")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache dtypes differ")
    return _Cache(N, B, H, d, _dtype_code(k_cache), float(k_scale), float(v_scale))


def _check(status: int, where: str):
    if status != PA_OK:
        raise PagedAttentionError(status, where)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, k_scale: float = 1.0,
                      v_scale: float = 1.0, stream=None) -> None:
    """Scatter key/value ``[T, Hkv, d]`` into their cache slots (``pa_reshape_and_cache``)."""
    torch = _torch()
    spec = cache_spec(k_cache, v_cache, k_scale, v_scale)
    if key.shape != value.shape or key.dtype != value.dtype:
        raise ValueError("key and value must match in shape and dtype")
    T = key.shape[0]
    if key.dim() != 3 or key.shape[1] != spec.num_kv_heads or key.shape[2] != spec.head_dim:
        raise ValueError(f"key must be [T, {spec.num_kv_heads}, {spec.head_dim}]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be int64 [T]")
    if T == 0:
        return
    st = library().pa_reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), _dtype_code(key), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), ctypes.byref(spec), _dev(slot_mapping, "slot_mapping"), T,
        _stream(stream))
    _check(st, "pa_reshape_and_cache")


def attention_workspace_size(k_cache, v_cache, num_q_heads: int, num_seqs: int, num_tokens: int,
                             max_seq_len: int, max_query_len: int) -> int:
    spec = cache_spec(k_cache, v_cache)
    out = ctypes.c_size_t(0)
    st = library().pa_attention_workspace_size(ctypes.byref(spec), num_q_heads, num_seqs,
                                               num_tokens, max_seq_len, max_query_len,
                                               ctypes.byref(out))
    _check(st, "pa_attention_workspace_size")
    return int(out.value)


def attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float, *,
              max_seq_len: Optional[int] = None, max_query_len: Optional[int] = None,
              out=None, workspace=None, k_scale: float = 1.0, v_scale: float = 1.0,
              prefix_len: int = 0, stream=None):
    """Paged attention of one mixed step (``pa_attention``); returns ``out``.

    max_seq_len / max_query_len are host-side upper bounds; if omitted they
    are read from the device tensors, which synchronises the stream.  With
    ``prefix_len`` > 0 every sequence shares its first prefix_len positions
    (the same blocks) and every query sits past them
    (``pa_attention_shared_prefix``: the prefix is attended once for all rows).
    """
    torch = _torch()
    spec = cache_spec(k_cache, v_cache, k_scale, v_scale)
    if q.dim() != 3 or q.shape[2] != spec.head_dim:
        raise ValueError(f"q must be [T, Hq, {spec.head_dim}]")
    T, Hq, _ = q.shape
    S = seq_lens.numel()
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("query_start_loc", query_start_loc)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if query_start_loc.numel() != S + 1 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("metadata shapes disagree")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if S else 0
    if max_query_len is None:
        max_query_len = int((query_start_loc[1:] - query_start_loc[:-1]).max().item()) if S else 0
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lib = library()
    need = ctypes.c_size_t(0)
    if prefix_len:
        _check(lib.pa_attention_shared_prefix_workspace_size(ctypes.byref(spec), Hq, S, T, max_seq_len,
                                                             max_query_len, int(prefix_len), ctypes.byref(need)),
               "pa_attention_shared_prefix_workspace_size")
    else:
        _check(lib.pa_attention_workspace_size(ctypes.byref(spec), Hq, S, T, max_seq_len,
                                               max_query_len, ctypes.byref(need)),
               "pa_attention_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=q.device)
    args = [_dev(q, "q"), _dtype_code(q), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            ctypes.byref(spec), _dev(block_tables, "block_tables"), block_tables.shape[1],
            _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), S, T, Hq,
            int(max_seq_len), int(max_query_len)]
    tail = [float(scale), _dev(out, "out"), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    if prefix_len:
        st = lib.pa_attention_shared_prefix(*args, int(prefix_len), *tail)
        _check(st, "pa_attention_shared_prefix")
    else:
        st = lib.pa_attention(*args, *tail)
        _check(st, "pa_attention")
    return out


def write_and_attend(key, value, slot_mapping, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                     scale: float, *, max_seq_len: int, max_query_len: int, out=None, workspace=None,
                     k_scale: float = 1.0, v_scale: float = 1.0, prefix_len: int = 0, stream=None):
    """The step's cache write of key/value ``[T_new, Hkv, d]`` into their
    slots, then paged attention of q (``pa_write_and_attend``: the two calls'
    result with one launch fewer; with ``prefix_len`` > 0 the attention is the
    shared-prefix one); returns ``out``."""
    torch = _torch()
    spec = cache_spec(k_cache, v_cache, k_scale, v_scale)
    if key.shape != value.shape or key.dtype != value.dtype:
        raise ValueError("key and value must match in shape and dtype")
    Tn = key.shape[0]
    if key.dim() != 3 or key.shape[1] != spec.num_kv_heads or key.shape[2] != spec.head_dim:
        raise ValueError(f"key must be [T, {spec.num_kv_heads}, {spec.head_dim}]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != Tn:
        raise ValueError("slot_mapping must be int64 [T]")
    if q.dim() != 3 or q.shape[2] != spec.head_dim:
        raise ValueError(f"q must be [T, Hq, {spec.head_dim}]")
    T, Hq, _ = q.shape
    S = seq_lens.numel()
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("query_start_loc", query_start_loc)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if query_start_loc.numel() != S + 1 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("metadata shapes disagree")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lib = library()
    if workspace is None:
        need = ctypes.c_size_t(0)
        if prefix_len:
            _check(lib.pa_attention_shared_prefix_workspace_size(ctypes.byref(spec), Hq, S, T, int(max_seq_len),
                                                                 int(max_query_len), int(prefix_len),
                                                                 ctypes.byref(need)),
                   "pa_attention_shared_prefix_workspace_size")
        else:
            _check(lib.pa_attention_workspace_size(ctypes.byref(spec), Hq, S, T, int(max_seq_len),
                                                   int(max_query_len), ctypes.byref(need)),
                   "pa_attention_workspace_size")
        workspace = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=q.device)
    kp = _dev(key, "key") if Tn else None
    vp = _dev(value, "value") if Tn else None
    sp = _dev(slot_mapping, "slot_mapping") if Tn else None
    st = lib.pa_write_and_attend(
        kp, vp, _dtype_code(key), sp, Tn, _dev(q, "q"), _dtype_code(q), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), ctypes.byref(spec), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), S, T, Hq, int(max_seq_len),
        int(max_query_len), int(prefix_len), float(scale), _dev(out, "out"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "pa_write_and_attend")
    return out


def bind_write_and_attend(key, value, slot_mapping, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                          scale: float, *, max_seq_len: int, max_query_len: int, out, workspace,
                          k_scale: float = 1.0, v_scale: float = 1.0, prefix_len: int = 0, stream=None):
    """``write_and_attend`` with its arguments marshalled once: returns a
    callable that issues the same ``pa_write_and_attend`` call (same
    buffers, stream and sizes) each time it is called, for loops that run
    one step shape over fixed buffers whose contents change between calls.
    The tensors must stay alive and in place while the callable is used."""
    torch = _torch()
    spec = cache_spec(k_cache, v_cache, k_scale, v_scale)
    Tn = key.shape[0]
    if key.shape != value.shape or key.dtype != value.dtype or slot_mapping.dtype != torch.int64 \
            or slot_mapping.numel() != Tn:
        raise ValueError("key, value and slot_mapping disagree")
    if key.dim() != 3 or key.shape[1] != spec.num_kv_heads or key.shape[2] != spec.head_dim:
        raise ValueError(f"key must be [T, {spec.num_kv_heads}, {spec.head_dim}]")
    if q.dim() != 3 or q.shape[2] != spec.head_dim or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must be [T, Hq, d] of one dtype")
    T, Hq, _ = q.shape
    S = seq_lens.numel()
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("query_start_loc", query_start_loc)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if query_start_loc.numel() != S + 1 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("metadata shapes disagree")
    fn = library().pa_write_and_attend
    args = (_dev(key, "key") if Tn else None, _dev(value, "value") if Tn else None, _dtype_code(key),
            _dev(slot_mapping, "slot_mapping") if Tn else None, Tn, _dev(q, "q"), _dtype_code(q),
            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ctypes.byref(spec),
            _dev(block_tables, "block_tables"), block_tables.shape[1], _dev(seq_lens, "seq_lens"),
            _dev(query_start_loc, "query_start_loc"), S, T, Hq, int(max_seq_len), int(max_query_len),
            int(prefix_len), float(scale), _dev(out, "out"), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))
    keep = (spec, key, value, slot_mapping, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, out,
            workspace)

    def call():
        _check(fn(*args), "pa_write_and_attend")
        return keep[10]

    return call


def attention_noalloc(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float, *,
                      max_seq_len: int, max_query_len: int, out, k_scale: float = 1.0, v_scale: float = 1.0,
                      stream=None):
    """``pa_attention_noalloc``: the step of :func:`attention`, with the work
    lists and partials in the library's static device scratch instead of a
    workspace.  Allocates nothing: the host bounds and ``out`` must be given
    (raises PagedAttentionError with PA_ERR_TOO_LARGE for a step whose
    workspace exceeds NOALLOC_SCRATCH_BYTES).  Calls that overlap on one
    device race; calls ordered on one stream do not."""
    torch = _torch()
    spec = cache_spec(k_cache, v_cache, k_scale, v_scale)
    if q.dim() != 3 or q.shape[2] != spec.head_dim:
        raise ValueError(f"q must be [T, Hq, {spec.head_dim}]")
    T, Hq, _ = q.shape
    S = seq_lens.numel()
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("query_start_loc", query_start_loc)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if query_start_loc.numel() != S + 1 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("metadata shapes disagree")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    st = library().pa_attention_noalloc(
        _dev(q, "q"), _dtype_code(q), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ctypes.byref(spec),
        _dev(block_tables, "block_tables"), block_tables.shape[1], _dev(seq_lens, "seq_lens"),
        _dev(query_start_loc, "query_start_loc"), S, T, Hq, int(max_seq_len), int(max_query_len), float(scale),
        _dev(out, "out"), _stream(stream))
    _check(st, "pa_attention_noalloc")
    return out


def preferred_block_size(head_dim: int, kv_dtype: int, q_dtype: int, group: int = 1) -> int:
    """Tokens per cache block the kernels run fastest with for this head dim,
    (q dtype, cache dtype) pairing and query group (q heads per kv head)
    (``pa_preferred_block_size``; dtype codes PA_F32 / PA_F16 / PA_BF16 /
    PA_FP8_E4M3)."""
    b = ctypes.c_int32(0)
    _check(library().pa_preferred_block_size(head_dim, kv_dtype, q_dtype, group, ctypes.byref(b)),
           "pa_preferred_block_size")
    return int(b.value)


def _pool(t, name):
    """Pointer of a pool tensor that the device can address: device memory or
    page-locked host memory (pin_memory)."""
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor or page-locked host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def copy_blocks(src_k, src_v, dst_k, dst_v, block_mapping, stream=None) -> None:
    """Copy whole blocks (``pa_copy_blocks``): for each row (s, t) of the int64
    ``[n, 2]`` device tensor ``block_mapping``, block t of (dst_k, dst_v)
    becomes block s of (src_k, src_v).  The same pool on both sides is a
    copy-on-write; a pinned host pool on one side is a swap."""
    torch = _torch()
    src = cache_spec(src_k, src_v)
    dst = cache_spec(dst_k, dst_v)
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be int64 [n, 2]")
    n = block_mapping.shape[0]
    if n == 0:
        return
    st = library().pa_copy_blocks(_pool(src_k, "src_k"), _pool(src_v, "src_v"), ctypes.byref(src),
                                  _pool(dst_k, "dst_k"), _pool(dst_v, "dst_v"), ctypes.byref(dst),
                                  _dev(block_mapping, "block_mapping"), n, _stream(stream))
    _check(st, "pa_copy_blocks")


def _i32(t, name, n=None, host_ok=False):
    torch = _torch()
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} elements")
    return _pool(t, name) if host_ok else _dev(t, name)


def apply_block_table_writes(block_table, rows, starts, offsets, values, stream=None) -> None:
    """Apply staged (row, start, values) runs to the device block table in
    place (``pa_apply_block_table_writes``).  The staging tensors may live in
    page-locked host memory; the kernel reads them there."""
    if block_table.dim() != 2:
        raise ValueError("block_table must be [max_reqs, max_blocks]")
    n = rows.numel()
    if n == 0 or values.numel() == 0:
        return
    st = library().pa_apply_block_table_writes(
        _i32(block_table, "block_table"), block_table.shape[0], block_table.shape[1],
        _i32(rows, "rows", n, True), _i32(starts, "starts", n, True), _i32(offsets, "offsets", n + 1, True),
        _i32(values, "values", None, True), n, values.numel(), _stream(stream))
    _check(st, "pa_apply_block_table_writes")


def prepare_step(block_table, idx_mapping, num_computed, num_scheduled, num_tokens: int, block_size: int,
                 out=None, stream=None):
    """Build the step's query_start_loc, seq_lens, positions, slot_mapping and
    block-table rows from persistent slot state (``pa_prepare_step``).
    Returns them as device tensors: new ones, or the five of ``out``."""
    torch = _torch()
    R = idx_mapping.numel()
    dev = block_table.device
    if out is None:
        out = (torch.empty(R + 1, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.int32, device=dev),
               torch.empty(num_tokens, dtype=torch.int64, device=dev),
               torch.empty(num_tokens, dtype=torch.int64, device=dev),
               torch.empty(R, block_table.shape[1], dtype=torch.int32, device=dev))
    qsl, lens, pos, slots, tables = out
    if (qsl.numel() != R + 1 or lens.numel() != R or pos.numel() != num_tokens or slots.numel() != num_tokens
            or tables.shape != (R, block_table.shape[1])):
        raise ValueError("prepare_step: output shapes disagree")
    if R == 0:
        qsl.zero_()
        return qsl, lens, pos, slots, tables
    st = library().pa_prepare_step(
        _i32(block_table, "block_table"), block_table.shape[0], block_table.shape[1],
        _i32(idx_mapping, "idx_mapping"), _i32(num_computed, "num_computed", block_table.shape[0]),
        _i32(num_scheduled, "num_scheduled", R), R, num_tokens, block_size, _dev(qsl, "qsl"), _dev(lens, "lens"),
        _dev(pos, "positions") if num_tokens else None, _dev(slots, "slot_mapping") if num_tokens else None,
        _dev(tables, "tables"), _stream(stream))
    _check(st, "pa_prepare_step")
    return qsl, lens, pos, slots, tables


def commit_step(num_computed, idx_mapping, num_scheduled, stream=None) -> None:
    """num_computed[idx_mapping[b]] += num_scheduled[b] on the device (``pa_commit_step``)."""
    R = idx_mapping.numel()
    if R == 0:
        return
    st = library().pa_commit_step(_i32(num_computed, "num_computed"), num_computed.numel(),
                                  _i32(idx_mapping, "idx_mapping"), _i32(num_scheduled, "num_scheduled", R), R,
                                  _stream(stream))
    _check(st, "pa_commit_step")


def set_attention_events(before, after) -> None:
    """Bracket the attention kernel with two hipEvent_t handles (ints), or None, None."""
    _check(library().pa_set_attention_events(before, after), "pa_set_attention_events")


def set_chunk_events(before, after) -> None:
    """Bracket the chunk (prefill) kernel with two hipEvent_t handles, or None, None."""
    _check(library().pa_set_chunk_events(before, after), "pa_set_chunk_events")


def set_prefix_events(before, after) -> None:
    """Bracket the shared-prefix pass with two hipEvent_t handles, or None, None."""
    _check(library().pa_set_prefix_events(before, after), "pa_set_prefix_events")


def check_metadata(k_cache, v_cache, block_tables, seq_lens, query_start_loc, num_tokens: int,
                   max_seq_len: int, max_query_len: int, stream=None):
    """Synchronous debug check of metadata contents; returns (ok, bad_seq)."""
    spec = cache_spec(k_cache, v_cache)
    bad = ctypes.c_int32(-1)
    st = library().pa_check_metadata(
        ctypes.byref(spec), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), seq_lens.numel(),
        num_tokens, max_seq_len, max_query_len, ctypes.byref(bad), _stream(stream))
    if st == PA_ERR_METADATA:
        return False, int(bad.value)
    _check(st, "pa_check_metadata")
    return True, -1
