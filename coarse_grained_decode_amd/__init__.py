"""SPICY-KV coarse-grained decode for MI355X (gfx950).

Thin Python binding over the C ABI in ``include/spicy.h``: argument
marshalling only (torch tensors -> device pointers, the current HIP stream).
Every step of coarsening and decoding runs in the library's HIP kernels
(``coarse_grained_decode_amd/libspicy.so``, built by
``python -m coarse_grained_decode_amd.build``).  There is no CPU fallback: if
the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "SpicyError", "PagedCache", "spicy_coarsen", "spicy_decode_attn",
    "spicy_coarsen_workspace_bytes", "spicy_decode_workspace_bytes", "spicy_decode_num_splits",
    "spicy_decode_attn_shared", "spicy_decode_shared_workspace_bytes",
    "spicy_policy", "spicy_policy_workspace_bytes",
    "spicy_decode_attn_multi", "spicy_decode_multi_workspace_bytes",
    "spicy_decode_attn_multi_noalloc", "spicy_decode_noalloc_max_bytes",
    "spicy_coarsen_weighted", "spicy_merge_level", "spicy_merge_workspace_bytes", "spicy_compact_range",
    "spicy_decode_plan",
    "spicy_status_string", "library_path", "load_library", "workspace", "device_error",
    "SPICY_F32", "SPICY_BF16", "PAGE_SIZE", "WORKSPACE_HEADER",
    "DEVERR_PAGE_ID", "DEVERR_CAPACITY", "DEVERR_SEGMENTS", "DEVERR_LENGTH", "DEVERR_SHARED", "DEVERR_POLICY",
    "DEVERR_TICKET",
]

SPICY_F32 = 0
SPICY_BF16 = 1
PAGE_SIZE = 16
WORKSPACE_HEADER = 256
DEVERR_PAGE_ID = 0x1
DEVERR_CAPACITY = 0x2
DEVERR_SEGMENTS = 0x4
DEVERR_LENGTH = 0x8
DEVERR_SHARED = 0x10
DEVERR_POLICY = 0x20
DEVERR_TICKET = 0x40

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspicy.so")
_lib = None


class SpicyError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {spicy_status_string(status)} ({status})")


class _Cache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("ab", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("s2", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libspicy.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m coarse_grained_decode_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(_LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    CP = ctypes.POINTER(_Cache)
    L.spicy_status_string.restype = ctypes.c_char_p
    L.spicy_status_string.argtypes = [ctypes.c_int]
    L.spicy_coarsen_workspace_bytes.restype = sz
    L.spicy_coarsen_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.spicy_coarsen.restype = ctypes.c_int
    L.spicy_coarsen.argtypes = [CP, P, P, i32, P, P, P, P, i32, P, i32, ctypes.c_double, P, i32,
                                P, P, P, sz, P]
    L.spicy_decode_plan.restype = ctypes.c_int
    L.spicy_decode_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, P]
    L.spicy_merge_workspace_bytes.restype = sz
    L.spicy_merge_workspace_bytes.argtypes = [i32, i32, i32]
    L.spicy_merge_level.restype = ctypes.c_int
    L.spicy_merge_level.argtypes = [CP, i32, ctypes.c_double, P, i32, P, P, i32, P, sz, P]
    L.spicy_compact_range.restype = ctypes.c_int
    L.spicy_compact_range.argtypes = [CP, i32, P, i32, P, P, P, P, P]
    L.spicy_coarsen_weighted.restype = ctypes.c_int
    L.spicy_coarsen_weighted.argtypes = [CP, P, P, i32, P, P, P, P, i32, P, P, i32, ctypes.c_double, P, i32,
                                         P, P, P, sz, P]
    L.spicy_decode_num_splits.restype = i32
    L.spicy_decode_num_splits.argtypes = [i32, i32, i32, i32]
    L.spicy_decode_workspace_bytes.restype = sz
    L.spicy_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.spicy_decode_attn.restype = ctypes.c_int
    L.spicy_decode_attn.argtypes = [CP, P, i32, P, i32, P, i32, P, P, P, sz, i32, P]
    L.spicy_decode_shared_workspace_bytes.restype = sz
    L.spicy_decode_shared_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.spicy_decode_attn_shared.restype = ctypes.c_int
    L.spicy_decode_attn_shared.argtypes = [CP, P, i32, P, i32, P, i32, i32, P, P, P, sz, i32, P]
    L.spicy_decode_multi_workspace_bytes.restype = sz
    L.spicy_decode_multi_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    L.spicy_decode_attn_multi.restype = ctypes.c_int
    L.spicy_decode_attn_multi.argtypes = [CP, P, i32, i32, P, i32, P, i32, i32, P, P, P, sz, i32, P]
    L.spicy_decode_noalloc_max_bytes.restype = sz
    L.spicy_decode_noalloc_max_bytes.argtypes = []
    L.spicy_decode_attn_multi_noalloc.restype = ctypes.c_int
    L.spicy_decode_attn_multi_noalloc.argtypes = [CP, P, i32, i32, P, i32, P, i32, i32, P, P, P, i32, P]
    L.spicy_policy_workspace_bytes.restype = sz
    L.spicy_policy_workspace_bytes.argtypes = [i32, i32]
    L.spicy_policy.restype = ctypes.c_int
    L.spicy_policy.argtypes = [P, P, i32, i32, i32, i32, P, i32, P, P, i32, i32, i32, i32, i32, i32,
                               P, P, P, P, sz, P]
    _lib = L
    return L


def spicy_status_string(status: int) -> str:
    return load_library().spicy_status_string(int(status)).decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.data_ptr() if t.numel() > 0 else None
    return int(t)


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream or None
        return None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream or None
    return int(stream) or None


_TORCH_DTYPE = {SPICY_BF16: torch.bfloat16, SPICY_F32: torch.float32}


def _check(t, name: str, dtype=None, shape=None, ndim=None, device=None, optional: bool = False):
    """Raise ValueError unless t is a contiguous tensor of the given dtype,
    shape (None entries match anything) or dimension count, on `device`.
    Runs before anything reaches the C ABI: a wrong dtype, layout or size
    would otherwise be read or written past the tensor's bytes."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: {t.dim()} dimensions, expected {ndim}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(n) != int(w) for n, w in zip(t.shape, shape)):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple('*' if w is None else w for w in shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, the cache is on {device}")


def _check_count(value: int, limit: int, name: str):
    if value < 0 or value > limit:
        raise ValueError(f"{name}: {value} outside [0, {limit}]")


@dataclass
class PagedCache:
    """Caller-owned paged compressed cache (device tensors in the library's layout).

    k    [num_pages, H_kv, d/8, 16, 8] rotated key rows, cut in 8-dim groups
    v    [num_pages, H_kv, d/8, 16, 8] value rows, the same way
    ab   [num_pages, H_kv, 16, 2]       (alpha, beta)
    meta [num_pages, H_kv, 16, 4] int32 {kind, mass, pos_sum lo, pos_sum hi} or None
    s2   [num_pages, H_kv, d/8, 16, 8] per-dimension variance (diagonal closure) or None
    """
    k: torch.Tensor
    v: torch.Tensor
    ab: torch.Tensor
    meta: torch.Tensor | None
    s2: torch.Tensor | None = None

    @staticmethod
    def empty(num_pages: int, H_kv: int, d: int, dtype: torch.dtype, device, meta: bool = True,
              fill: float | None = None, diag: bool = False) -> "PagedCache":
        mk = torch.empty if fill is None else (lambda *s, **kw: torch.full(s, fill, **kw))
        k = mk(num_pages, H_kv, d // 8, PAGE_SIZE, 8, dtype=dtype, device=device)
        v = mk(num_pages, H_kv, d // 8, PAGE_SIZE, 8, dtype=dtype, device=device)
        ab = mk(num_pages, H_kv, PAGE_SIZE, 2, dtype=dtype, device=device)
        mt = torch.zeros(num_pages, H_kv, PAGE_SIZE, 4, dtype=torch.int32, device=device) if meta else None
        s2 = mk(num_pages, H_kv, d // 8, PAGE_SIZE, 8, dtype=dtype, device=device) if diag else None
        return PagedCache(k, v, ab, mt, s2)

    @property
    def num_pages(self) -> int:
        return int(self.k.shape[0])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.k.shape[2] * self.k.shape[4])

    @property
    def dtype_code(self) -> int:
        if self.k.dtype == torch.bfloat16:
            return SPICY_BF16
        if self.k.dtype == torch.float32:
            return SPICY_F32
        raise ValueError(f"unsupported cache dtype {self.k.dtype}")

    def check(self):
        """The pool tensors' dtypes, shapes and devices agree."""
        dt = _TORCH_DTYPE[self.dtype_code]
        P, H, d = self.num_pages, self.num_kv_heads, self.head_dim
        dev = self.k.device
        _check(self.k, "cache.k", dt, (P, H, d // 8, PAGE_SIZE, 8))
        _check(self.v, "cache.v", dt, (P, H, d // 8, PAGE_SIZE, 8), device=dev)
        _check(self.ab, "cache.ab", dt, (P, H, PAGE_SIZE, 2), device=dev)
        _check(self.meta, "cache.meta", torch.int32, (P, H, PAGE_SIZE, 4), device=dev, optional=True)
        _check(self.s2, "cache.s2", dt, (P, H, d // 8, PAGE_SIZE, 8), device=dev, optional=True)
        return dev

    def struct(self) -> _Cache:
        return _Cache(self.dtype_code, self.num_kv_heads, self.head_dim, self.num_pages,
                      _ptr(self.k), _ptr(self.v), _ptr(self.ab), _ptr(self.meta), _ptr(self.s2))


def spicy_coarsen_workspace_bytes(B: int, n_seg: int, total_tokens: int, num_kv_heads: int, head_dim: int,
                                  dtype: int) -> int:
    return int(load_library().spicy_coarsen_workspace_bytes(B, n_seg, total_tokens, num_kv_heads, head_dim,
                                                            dtype))


def spicy_decode_num_splits(B: int, num_kv_heads: int, max_pages_per_seq: int, num_splits: int = 0) -> int:
    return int(load_library().spicy_decode_num_splits(B, num_kv_heads, max_pages_per_seq, num_splits))


def spicy_decode_workspace_bytes(B: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                 max_pages_per_seq: int, num_splits: int = 0) -> int:
    return int(load_library().spicy_decode_workspace_bytes(B, num_q_heads, num_kv_heads, head_dim,
                                                           max_pages_per_seq, num_splits))


def spicy_coarsen(cache: PagedCache, k_pre, v, seq_offsets, pos_base, seg_offsets, seq_seg_ptr,
                  protected_mask, rope_base: float, page_table, entry_start, lengths_out,
                  workspace, stream=None, *, total_tokens: int | None = None, n_seg: int | None = None,
                  B: int | None = None, max_pages_per_seq: int | None = None) -> None:
    """spicy_coarsen through the C ABI (see include/spicy.h)."""
    L = load_library()
    B, n_seg, total_tokens, max_pages = _check_coarsen(cache, k_pre, v, seq_offsets, pos_base, seg_offsets,
                                                       seq_seg_ptr, protected_mask, page_table, entry_start,
                                                       lengths_out, workspace, total_tokens, n_seg, B,
                                                       max_pages_per_seq)
    st = cache.struct()
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    rc = L.spicy_coarsen(ctypes.byref(st), _ptr(k_pre), _ptr(v), total_tokens, _ptr(seq_offsets),
                         _ptr(pos_base), _ptr(seg_offsets), _ptr(seq_seg_ptr), n_seg, _ptr(protected_mask),
                         B, float(rope_base), _ptr(page_table), max_pages, _ptr(entry_start),
                         _ptr(lengths_out), _ptr(workspace), ws_bytes, _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_coarsen")


def _check_coarsen(cache, k_pre, v, seq_offsets, pos_base, seg_offsets, seq_seg_ptr, protected_mask, page_table,
                   entry_start, lengths_out, workspace, total_tokens, n_seg, B, max_pages_per_seq):
    """Validate spicy_coarsen's tensors; returns (B, n_seg, total_tokens, max_pages)."""
    dev = cache.check()
    dt = _TORCH_DTYPE[cache.dtype_code]
    H, d = cache.num_kv_heads, cache.head_dim
    _check(k_pre, "k_pre", dt, (None, H, d), device=dev)
    _check(v, "v", dt, tuple(k_pre.shape), device=dev)
    _check(protected_mask, "protected_mask", torch.uint8, (k_pre.shape[0], H), device=dev)
    _check(seq_offsets, "seq_offsets", torch.int32, ndim=1, device=dev)
    _check(seg_offsets, "seg_offsets", torch.int32, ndim=1, device=dev)
    _check(seq_seg_ptr, "seq_seg_ptr", torch.int32, tuple(seq_offsets.shape), device=dev)
    _check(page_table, "page_table", torch.int32, ndim=2, device=dev)
    _check(workspace, "workspace", ndim=1, device=dev)
    nb = int(seq_offsets.shape[0]) - 1
    B = nb if B is None else B
    _check_count(B, max(nb, 0), "B")
    _check(pos_base, "pos_base", torch.int32, (None,), device=dev, optional=True)
    _check(entry_start, "entry_start", torch.int32, (None,), device=dev, optional=True)
    _check(lengths_out, "lengths_out", torch.int32, (None,), device=dev)
    for t, nm in ((pos_base, "pos_base"), (entry_start, "entry_start"), (lengths_out, "lengths_out")):
        if t is not None and t.shape[0] < B:
            raise ValueError(f"{nm}: {t.shape[0]} entries for {B} sequences")
    if page_table.shape[0] < B:
        raise ValueError(f"page_table: {page_table.shape[0]} rows for {B} sequences")
    n_seg = int(seg_offsets.shape[0]) - 1 if n_seg is None else n_seg
    _check_count(n_seg, int(seg_offsets.shape[0]) - 1, "n_seg")
    total_tokens = int(k_pre.shape[0]) if total_tokens is None else total_tokens
    _check_count(total_tokens, int(k_pre.shape[0]), "total_tokens")
    max_pages = int(page_table.shape[1]) if max_pages_per_seq is None else max_pages_per_seq
    _check_count(max_pages, int(page_table.shape[1]), "max_pages_per_seq")
    return B, n_seg, total_tokens, max_pages


def _check_decode(cache, q, page_table, lengths, o, lse, workspace, n_q, B, max_pages_per_seq):
    """Validate a decode call's tensors: q [B, (n_q,) H_q, d] in the cache's
    dtype, o float32 of q's shape, lse float32 [B, (n_q,) H_q]; returns
    (B, H_q, max_pages)."""
    dev = cache.check()
    dt = _TORCH_DTYPE[cache.dtype_code]
    d = cache.head_dim
    lead = (None, n_q) if n_q is not None else (None,)
    _check(q, "q", dt, lead + (None, d), device=dev)
    _check(o, "o", torch.float32, tuple(q.shape), device=dev)
    _check(lse, "lse", torch.float32, tuple(q.shape[:-1]), device=dev)
    _check(page_table, "page_table", torch.int32, ndim=2, device=dev)
    _check(lengths, "lengths", torch.int32, (None,), device=dev)
    _check(workspace, "workspace", ndim=1, device=dev)
    nb = int(q.shape[0])
    B = nb if B is None else B
    _check_count(B, nb, "B")
    if page_table.shape[0] < B or lengths.shape[0] < B:
        raise ValueError(f"page_table / lengths: fewer rows than the {B} sequences")
    max_pages = int(page_table.shape[1]) if max_pages_per_seq is None else max_pages_per_seq
    _check_count(max_pages, int(page_table.shape[1]), "max_pages_per_seq")
    return B, int(q.shape[-2]), max_pages


def spicy_decode_plan(B: int, num_q_heads: int, num_kv_heads: int, max_pages_per_seq: int,
                      shared_prefix_pages: int = 0, num_splits: int = 0, num_q_tokens: int = 1) -> dict:
    """spicy_decode_plan: the decode's split-K plan for these sizes."""
    out = (ctypes.c_int32 * 4)()
    rc = load_library().spicy_decode_plan(B, num_q_heads, num_kv_heads, max_pages_per_seq, shared_prefix_pages,
                                          num_splits, num_q_tokens, out)
    if rc != 0:
        raise SpicyError(rc, "spicy_decode_plan")
    return dict(prefix_chunks=out[0], prefix_chunk_pages=out[1], private_splits=out[2],
                private_pages_per_split=out[3])


def spicy_merge_workspace_bytes(B: int, num_kv_heads: int, max_range: int) -> int:
    return int(load_library().spicy_merge_workspace_bytes(B, num_kv_heads, max_range))


def spicy_merge_level(cache: PagedCache, rope_base: float, page_table, entry_begin, entry_end, max_range: int,
                      workspace, stream=None, *, B: int | None = None,
                      max_pages_per_seq: int | None = None) -> None:
    """spicy_merge_level through the C ABI (see include/spicy.h): one level of
    the dyadic merge over entries [entry_begin[b], entry_end[b]) in place."""
    L = load_library()
    dev = cache.check()
    _check(page_table, "page_table", torch.int32, ndim=2, device=dev)
    _check(entry_begin, "entry_begin", torch.int32, (None,), device=dev)
    _check(entry_end, "entry_end", torch.int32, tuple(entry_begin.shape), device=dev)
    _check(workspace, "workspace", ndim=1, device=dev)
    B = int(entry_begin.shape[0]) if B is None else B
    _check_count(B, int(entry_begin.shape[0]), "B")
    if page_table.shape[0] < B:
        raise ValueError(f"page_table: {page_table.shape[0]} rows for {B} sequences")
    max_pages = int(page_table.shape[1]) if max_pages_per_seq is None else max_pages_per_seq
    _check_count(max_pages, int(page_table.shape[1]), "max_pages_per_seq")
    st = cache.struct()
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    rc = L.spicy_merge_level(ctypes.byref(st), B, float(rope_base), _ptr(page_table), max_pages, _ptr(entry_begin),
                             _ptr(entry_end), int(max_range), _ptr(workspace), ws_bytes, _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_merge_level")


def spicy_compact_range(cache: PagedCache, page_table, entry_begin, lengths, lengths_out, device_error,
                        stream=None, *, B: int | None = None, max_pages_per_seq: int | None = None) -> None:
    """spicy_compact_range through the C ABI (see include/spicy.h): per
    sequence and KV head the non-null entries of [entry_begin[b], lengths[b])
    move, in order, to the front of the range; lengths_out[b] gets the new
    length.  device_error: int32 device tensor whose first element receives
    SPICY_DEVERR_* bits."""
    L = load_library()
    dev = cache.check()
    _check(page_table, "page_table", torch.int32, ndim=2, device=dev)
    _check(entry_begin, "entry_begin", torch.int32, (None,), device=dev)
    _check(lengths, "lengths", torch.int32, tuple(entry_begin.shape), device=dev)
    _check(lengths_out, "lengths_out", torch.int32, tuple(entry_begin.shape), device=dev)
    _check(device_error, "device_error", torch.int32, ndim=1, device=dev)
    if device_error.numel() < 1:
        raise ValueError("device_error: needs one int32")
    if lengths_out.data_ptr() in (lengths.data_ptr(), entry_begin.data_ptr()):
        raise ValueError("lengths_out: must be a tensor of its own (not lengths or entry_begin)")
    B = int(entry_begin.shape[0]) if B is None else B
    _check_count(B, int(entry_begin.shape[0]), "B")
    if page_table.shape[0] < B:
        raise ValueError(f"page_table: {page_table.shape[0]} rows for {B} sequences")
    max_pages = int(page_table.shape[1]) if max_pages_per_seq is None else max_pages_per_seq
    _check_count(max_pages, int(page_table.shape[1]), "max_pages_per_seq")
    st = cache.struct()
    rc = L.spicy_compact_range(ctypes.byref(st), B, _ptr(page_table), max_pages, _ptr(entry_begin), _ptr(lengths),
                               _ptr(lengths_out), _ptr(device_error), _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_compact_range")


def spicy_coarsen_weighted(cache: PagedCache, k_pre, v, seq_offsets, pos_base, seg_offsets, seq_seg_ptr,
                           protected_mask, token_weight, rope_base: float, page_table, entry_start, lengths_out,
                           workspace, stream=None, *, total_tokens: int | None = None, n_seg: int | None = None,
                           B: int | None = None, max_pages_per_seq: int | None = None) -> None:
    """spicy_coarsen_weighted through the C ABI (see include/spicy.h);
    token_weight: int64 device tensor [total_tokens]."""
    L = load_library()
    B, n_seg, total_tokens, max_pages = _check_coarsen(cache, k_pre, v, seq_offsets, pos_base, seg_offsets,
                                                       seq_seg_ptr, protected_mask, page_table, entry_start,
                                                       lengths_out, workspace, total_tokens, n_seg, B,
                                                       max_pages_per_seq)
    _check(token_weight, "token_weight", torch.int64, (None,), device=k_pre.device)
    if token_weight.shape[0] < total_tokens:
        raise ValueError(f"token_weight: {token_weight.shape[0]} weights for {total_tokens} tokens")
    st = cache.struct()
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    rc = L.spicy_coarsen_weighted(ctypes.byref(st), _ptr(k_pre), _ptr(v), total_tokens, _ptr(seq_offsets),
                                  _ptr(pos_base), _ptr(seg_offsets), _ptr(seq_seg_ptr), n_seg,
                                  _ptr(protected_mask), _ptr(token_weight), B, float(rope_base), _ptr(page_table),
                                  max_pages, _ptr(entry_start), _ptr(lengths_out), _ptr(workspace), ws_bytes,
                                  _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_coarsen_weighted")


def spicy_decode_attn(cache: PagedCache, q, page_table, lengths, o, lse, workspace,
                      num_splits: int = 0, stream=None, *, B: int | None = None,
                      num_q_heads: int | None = None, max_pages_per_seq: int | None = None) -> None:
    """spicy_decode_attn through the C ABI (see include/spicy.h)."""
    L = load_library()
    B, H_q, max_pages = _check_decode(cache, q, page_table, lengths, o, lse, workspace, None, B, max_pages_per_seq)
    if num_q_heads is not None and num_q_heads != H_q:
        raise ValueError(f"num_q_heads {num_q_heads} differs from q's {H_q}")
    st = cache.struct()
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    rc = L.spicy_decode_attn(ctypes.byref(st), _ptr(q), H_q, _ptr(page_table), max_pages, _ptr(lengths), B,
                             _ptr(o), _ptr(lse), _ptr(workspace), ws_bytes, int(num_splits), _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_decode_attn")


def spicy_decode_shared_workspace_bytes(B: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                        max_pages_per_seq: int, shared_prefix_pages: int,
                                        num_splits: int = 0) -> int:
    return int(load_library().spicy_decode_shared_workspace_bytes(B, num_q_heads, num_kv_heads, head_dim,
                                                                  max_pages_per_seq, shared_prefix_pages,
                                                                  num_splits))


def spicy_decode_attn_shared(cache: PagedCache, q, page_table, lengths, shared_prefix_pages: int, o, lse,
                             workspace, num_splits: int = 0, stream=None, *, B: int | None = None,
                             num_q_heads: int | None = None, max_pages_per_seq: int | None = None) -> None:
    """spicy_decode_attn_shared through the C ABI (see include/spicy.h)."""
    L = load_library()
    B, H_q, max_pages = _check_decode(cache, q, page_table, lengths, o, lse, workspace, None, B, max_pages_per_seq)
    if num_q_heads is not None and num_q_heads != H_q:
        raise ValueError(f"num_q_heads {num_q_heads} differs from q's {H_q}")
    st = cache.struct()
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    rc = L.spicy_decode_attn_shared(ctypes.byref(st), _ptr(q), H_q, _ptr(page_table), max_pages,
                                    _ptr(lengths), B, int(shared_prefix_pages), _ptr(o), _ptr(lse),
                                    _ptr(workspace), ws_bytes, int(num_splits), _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_decode_attn_shared")


def spicy_decode_multi_workspace_bytes(B: int, num_q_tokens: int, num_q_heads: int, num_kv_heads: int,
                                       head_dim: int, max_pages_per_seq: int, shared_prefix_pages: int = 0,
                                       num_splits: int = 0) -> int:
    return int(load_library().spicy_decode_multi_workspace_bytes(B, num_q_tokens, num_q_heads, num_kv_heads,
                                                                 head_dim, max_pages_per_seq,
                                                                 shared_prefix_pages, num_splits))


def spicy_decode_attn_multi(cache: PagedCache, q, page_table, lengths, shared_prefix_pages: int, o, lse,
                            workspace, num_splits: int = 0, stream=None, *, B: int | None = None,
                            max_pages_per_seq: int | None = None) -> None:
    """spicy_decode_attn_multi through the C ABI (see include/spicy.h):
    q [B, n_q, H_q, d] -> o [B, n_q, H_q, d], lse [B, n_q, H_q]."""
    L = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q: expected a [B, n_q, H_q, d] tensor")
    n_q = int(q.shape[1])
    B, H_q, max_pages = _check_decode(cache, q, page_table, lengths, o, lse, workspace, n_q, B, max_pages_per_seq)
    st = cache.struct()
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    rc = L.spicy_decode_attn_multi(ctypes.byref(st), _ptr(q), n_q, H_q, _ptr(page_table), max_pages,
                                   _ptr(lengths), B, int(shared_prefix_pages), _ptr(o), _ptr(lse),
                                   _ptr(workspace), ws_bytes, int(num_splits), _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_decode_attn_multi")


def spicy_decode_noalloc_max_bytes() -> int:
    return int(load_library().spicy_decode_noalloc_max_bytes())


def spicy_decode_attn_multi_noalloc(cache: PagedCache, q, page_table, lengths, shared_prefix_pages: int, o, lse,
                                    device_error=None, num_splits: int = 0, stream=None, *, B: int | None = None,
                                    max_pages_per_seq: int | None = None) -> None:
    """spicy_decode_attn_multi_noalloc through the C ABI (see include/spicy.h):
    spicy_decode_attn_multi without a workspace; device_error: an int32
    device tensor of one element (the sticky error word) or None."""
    L = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q: expected a [B, n_q, H_q, d] tensor")
    n_q = int(q.shape[1])
    ws_stub = torch.empty(1, dtype=torch.int32, device=q.device)
    B, H_q, max_pages = _check_decode(cache, q, page_table, lengths, o, lse, ws_stub, n_q, B, max_pages_per_seq)
    _check(device_error, "device_error", torch.int32, (None,), device=q.device, optional=True)
    st = cache.struct()
    rc = L.spicy_decode_attn_multi_noalloc(ctypes.byref(st), _ptr(q), n_q, H_q, _ptr(page_table), max_pages,
                                           _ptr(lengths), B, int(shared_prefix_pages), _ptr(o), _ptr(lse),
                                           _ptr(device_error), int(num_splits), _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_decode_attn_multi_noalloc")


def spicy_policy_workspace_bytes(total_tokens: int, num_kv_heads: int) -> int:
    return int(load_library().spicy_policy_workspace_bytes(total_tokens, num_kv_heads))


def spicy_policy(k_pre, v, seq_offsets, proj_ptr, proj_idx, n_segments: int, n_landmarks: int, sink: int,
                 recent: int, seg_offsets, seq_seg_ptr, protected_mask, workspace, stream=None, *,
                 B: int | None = None, total_tokens: int | None = None) -> None:
    """spicy_policy through the C ABI (see include/spicy.h): segment slots and
    protection mask of a chunk (k_pre, v: [total_tokens, H, d] bf16)."""
    L = load_library()
    _check(k_pre, "k_pre", torch.bfloat16, ndim=3)
    dev = k_pre.device
    _check(v, "v", torch.bfloat16, tuple(k_pre.shape), device=dev)
    H, d = int(k_pre.shape[1]), int(k_pre.shape[2])
    _check(seq_offsets, "seq_offsets", torch.int32, ndim=1, device=dev)
    _check(proj_ptr, "proj_ptr", torch.int32, ndim=1, device=dev)
    _check(proj_idx, "proj_idx", torch.int32, ndim=1, device=dev)
    _check(workspace, "workspace", ndim=1, device=dev)
    nb = int(seq_offsets.shape[0]) - 1
    B = nb if B is None else B
    _check_count(B, max(nb, 0), "B")
    _check(seg_offsets, "seg_offsets", torch.int32, (B * int(n_segments) + 1,), device=dev)
    _check(seq_seg_ptr, "seq_seg_ptr", torch.int32, (B + 1,), device=dev)
    _check(protected_mask, "protected_mask", torch.uint8, (k_pre.shape[0], H), device=dev)
    total_tokens = int(k_pre.shape[0]) if total_tokens is None else total_tokens
    _check_count(total_tokens, int(k_pre.shape[0]), "total_tokens")
    dtype = SPICY_BF16
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    rc = L.spicy_policy(_ptr(k_pre), _ptr(v), total_tokens, H, d, dtype, _ptr(seq_offsets), B,
                        _ptr(proj_ptr), _ptr(proj_idx), int(proj_ptr.shape[0] - 1), int(proj_idx.numel()),
                        int(n_segments), int(n_landmarks), int(sink), int(recent), _ptr(seg_offsets),
                        _ptr(seq_seg_ptr), _ptr(protected_mask), _ptr(workspace), ws_bytes, _stream(stream))
    if rc != 0:
        raise SpicyError(rc, "spicy_policy")


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zeroed workspace buffer (the sticky error word starts at zero)."""
    return torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=device)


def device_error(ws: torch.Tensor) -> int:
    """Read (synchronously) the sticky device error word of a workspace."""
    return int(ws[0].item())
