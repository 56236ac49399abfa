"""CPU oracle for SPICY-KV coarsen + decode — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``coarse_grained_decode_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``spicy_oracle.c`` (plain C, double precision, one
step at a time as the pages define it).  This module only marshals numpy
arrays into that library and splits the batch over host threads.

Parity: coarsening and decoding are pinned by the tests in ``tests/`` against
closed forms, library routines and invariants (see the test docstrings).  The
agreement with the pages' own quality results (RULER recall, the demo page's
simulator table) is *parity unpinned*: the pages print no values to compare.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "spicy_oracle.c")

DT = {"f32": 0, "bf16": 1, "f64": 2}
NP = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}
META_DTYPE = np.dtype([("kind", "<i4"), ("mass", "<i4"), ("pos_sum", "<i8")])
PAGE = 16

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no contraction)."""
    if force or not os.path.exists(LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
               "-fno-fast-math", "-shared", "-fPIC", "-o", LIB, SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            L = ctypes.CDLL(LIB)
            P = ctypes.c_void_p
            i32 = ctypes.c_int32
            L.oracle_coarsen.restype = ctypes.c_int
            L.oracle_coarsen.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, P, P, P, P, P, P, P,
                                         i32, ctypes.c_double, P, P, P, P, i32, P, i32, P, P, i32, i32]
            L.oracle_decode.restype = ctypes.c_int
            L.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, i32, P, P, P, P, i32,
                                        P, i32, P, i32, P, P, i32, i32]
            L.oracle_coarsen_diag.restype = ctypes.c_int
            L.oracle_coarsen_diag.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, P, P, P, P, P, P, P,
                                              i32, ctypes.c_double, P, P, P, P, P, i32, P, i32, P, P, i32, i32]
            L.oracle_coarsen_weighted.restype = ctypes.c_int
            L.oracle_coarsen_weighted.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, P, P, P, P, P, P, P, P,
                                                  i32, ctypes.c_double, P, P, P, P, P, i32, P, i32, P, P, i32, i32]
            L.oracle_merge_level.restype = ctypes.c_int
            L.oracle_merge_level.argtypes = [ctypes.c_int, i32, i32, P, P, P, P, P, i32, P, i32, P, P, i32,
                                             ctypes.c_double, i32, i32]
            L.oracle_compact_range.restype = ctypes.c_int
            L.oracle_compact_range.argtypes = [ctypes.c_int, i32, i32, P, P, P, P, P, i32, P, i32, P, P, i32, P,
                                               i32, i32]
            L.oracle_decode_heads.restype = ctypes.c_int
            L.oracle_decode_heads.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, i32, P, P, P, P, P, i32,
                                              P, i32, P, i32, P, P, i32, i32, i32, i32]
            L.oracle_decode_diag.restype = ctypes.c_int
            L.oracle_decode_diag.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, i32, P, P, P, P, P, i32,
                                             P, i32, P, i32, P, P, i32, i32]
            L.oracle_bf16_round.restype = ctypes.c_uint16
            L.oracle_bf16_round.argtypes = [ctypes.c_double]
            L.oracle_bf16_value.restype = ctypes.c_double
            L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
            L.oracle_rope.restype = None
            L.oracle_rope.argtypes = [P, P, i32, ctypes.c_double, ctypes.c_double]
            L.oracle_fix16.restype = ctypes.c_int64
            L.oracle_fix16.argtypes = [ctypes.c_uint16]
            L.oracle_isqrt_u128.restype = ctypes.c_uint64
            L.oracle_isqrt_u128.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
            L.oracle_policy.restype = ctypes.c_int
            L.oracle_policy.argtypes = [i32, i32, P, P, P, i32, P, P, i32, i32, i32, i32, i32,
                                        P, P, P, P, P]
            _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _chunks(B, threads):
    threads = max(1, min(threads, B))
    step = -(-B // threads) if B else 1
    return [(s, min(B, s + step)) for s in range(0, B, step)] or [(0, 0)]


def default_threads() -> int:
    """Host threads: the process's affinity set, capped by OMP_NUM_THREADS
    when the environment sets it (each GPU process's share of the host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def chunk_width(d: int) -> int:
    """Dims per group of the key/value page layout: min(8, d)."""
    return d if d < 8 else 8


def rows(x: np.ndarray) -> np.ndarray:
    """[P, H, d/W, 16, W] key or value pages as [P, H, 16, d] entry rows (copy)."""
    P, H, C, S, W = x.shape
    return np.ascontiguousarray(x.transpose(0, 1, 3, 2, 4)).reshape(P, H, S, C * W)


class Cache:
    """Host copy of a paged compressed cache in the library's layout:
    k, v [P, H, d/W, 16, W] (entry rows cut in groups of W = min(8, d) dims),
    ab [P, H, 16, 2], meta [P, H, 16]."""

    def __init__(self, store: str, num_pages: int, H_kv: int, d: int, fill: bool = True, diag: bool = False):
        self.store, self.num_pages, self.H_kv, self.d = store, num_pages, H_kv, d
        dt = NP[store]
        W = chunk_width(d)
        self.k = np.empty((num_pages, H_kv, d // W, PAGE, W), dtype=dt)
        self.v = np.empty((num_pages, H_kv, d // W, PAGE, W), dtype=dt)
        self.ab = np.empty((num_pages, H_kv, PAGE, 2), dtype=dt)
        self.meta = np.zeros((num_pages, H_kv, PAGE), dtype=META_DTYPE)
        # the diagonal closure's per-dimension variance sidecar, laid out like k
        self.s2 = np.empty((num_pages, H_kv, d // W, PAGE, W), dtype=dt) if diag else None
        if fill:  # recognisable garbage so that unwritten slots never look valid
            for a in (self.k, self.v, self.ab) + ((self.s2,) if diag else ()):
                if store == "bf16":
                    a.fill(0x7FC1)
                else:
                    a.fill(np.nan)
            self.meta["kind"] = -1


def coarsen(call, cache: Cache, in_dtype: str | None = None, threads: int | None = None,
            token_weight: np.ndarray | None = None) -> np.ndarray:
    """Run oracle_coarsen for one CoarsenCall into `cache` (oracle_coarsen_diag
    when the cache carries the diagonal-variance sidecar; oracle_coarsen_weighted
    with per-token weights, int64 [total_tokens]); returns lengths_out."""
    L = lib()
    in_dtype = in_dtype or call.dtype
    k = np.ascontiguousarray(call.k)
    v = np.ascontiguousarray(call.v)
    lengths = np.zeros(call.B, dtype=np.int32)
    tw = None if token_weight is None else np.ascontiguousarray(token_weight, dtype=np.int64)
    if tw is not None and tw.shape != (k.shape[0],):
        raise ValueError("token_weight needs one int64 per token")
    args_fixed = dict()
    rcs = []

    def run(rng):
        b0, b1 = rng
        head = (DT[in_dtype], DT[cache.store], call.H_kv, call.d, _p(k), _p(v),
                _p(call.seq_offsets), _p(call.pos_base), _p(call.seg_offsets),
                _p(call.seq_seg_ptr), _p(call.mask), call.B, call.rope_base,
                _p(cache.k), _p(cache.v), _p(cache.ab), _p(cache.meta))
        tail = (cache.num_pages, _p(call.page_table), call.max_pages, _p(call.entry_start), _p(lengths), b0, b1)
        if tw is not None:
            rc = L.oracle_coarsen_weighted(*head[:11], _p(tw), *head[11:], _p(cache.s2), *tail)
        elif cache.s2 is None:
            rc = L.oracle_coarsen(*head, *tail)
        else:
            rc = L.oracle_coarsen_diag(*head, _p(cache.s2), *tail)
        rcs.append(rc)

    del args_fixed
    chunks = _chunks(call.B, threads or default_threads())
    if len(chunks) == 1:
        run(chunks[0])
    else:
        with ThreadPoolExecutor(len(chunks)) as ex:
            list(ex.map(run, chunks))
    if any(rc != 0 for rc in rcs):
        raise ValueError(f"oracle_coarsen failed: codes {sorted(set(rcs))}")
    return lengths


def decode(q: np.ndarray, q_dtype: str, cache: Cache, H_q: int, page_table: np.ndarray,
           lengths: np.ndarray, threads: int | None = None):
    """Run the oracle decode (with the diagonal closure on a cache with the
    diagonal sidecar), one (sequence, KV head) per work item over `threads`
    host threads; returns (o [B, H_q, d] float64, lse [B, H_q] float64)."""
    L = lib()
    q = np.ascontiguousarray(q)
    B = int(q.shape[0])
    d = cache.d
    if q.ndim != 3 or q.shape[1:] != (H_q, d) or q.dtype != NP[q_dtype]:
        raise ValueError(f"q must be [B, {H_q}, {d}] of {q_dtype} storage, got {q.shape} {q.dtype}")
    if np.shape(lengths) != (B,) or np.shape(page_table)[0] != B:
        raise ValueError("page_table and lengths need one row per sequence")
    o = np.zeros((B, H_q, d), dtype=np.float64)
    lse = np.zeros((B, H_q), dtype=np.float64)
    table = np.ascontiguousarray(page_table, dtype=np.int32)
    lens = np.ascontiguousarray(lengths, dtype=np.int32)
    rcs = []
    G = H_q // cache.H_kv if cache.H_kv > 0 and H_q % cache.H_kv == 0 else H_q

    def run(unit):
        # one work item: the query heads of one KV head of one sequence
        b, h = unit
        rcs.append(L.oracle_decode_heads(DT[q_dtype], DT[cache.store], H_q, cache.H_kv, d, _p(q), _p(cache.k),
                                         _p(cache.v), _p(cache.ab), _p(cache.s2), cache.num_pages, _p(table),
                                         int(table.shape[1]), _p(lens), B, _p(o), _p(lse), b, b + 1,
                                         h * G, (h + 1) * G))

    units = [(b, h) for b in range(B) for h in range(H_q // G)]
    n = max(1, min(threads or default_threads(), len(units)))
    if n == 1:
        for u in units:
            run(u)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(run, units))
    if any(rc != 0 for rc in rcs):
        raise ValueError(f"oracle_decode failed: codes {sorted(set(rcs))}")
    return o, lse


def decode_multi(q: np.ndarray, q_dtype: str, cache: Cache, page_table: np.ndarray, lengths: np.ndarray,
                 threads: int | None = None):
    """Several query tokens per sequence: q [B, n_q, H_q, d].  Every token's
    rows attend to its sequence's entries exactly as a single query does
    (the decode definition applied per query row), so this is oracle_decode
    over the B * n_q (sequence, token) rows, each with its sequence's page
    table row and length.  Returns (o [B, n_q, H_q, d], lse [B, n_q, H_q])."""
    B, n_q, H_q, d = q.shape
    qq = np.ascontiguousarray(q).reshape(B * n_q, H_q, d)
    table = np.repeat(np.asarray(page_table), n_q, axis=0)
    lens = np.repeat(np.asarray(lengths), n_q)
    o, lse = decode(qq, q_dtype, cache, H_q, table, lens, threads)
    return o.reshape(B, n_q, H_q, d), lse.reshape(B, n_q, H_q)


def run_workload(wl, store: str | None = None, threads: int | None = None, diag: bool = False):
    """Coarsen every call of a workload (setup calls, then the step call once)
    into a fresh cache and decode its queries.  Returns (cache, lengths, o, lse).
    diag: the cache carries the diagonal closure's variance sidecar."""
    store = store or wl.dtype
    cache = Cache(store, wl.num_pages, wl.H_kv, wl.d, diag=diag)
    lengths = None
    for call in wl.calls:
        lengths = coarsen(call, cache, threads=threads)
    o, lse = decode(wl.q, wl.dtype, cache, wl.H_q, wl.page_table, lengths, threads=threads)
    return cache, lengths, o, lse


def merge_level(cache: Cache, page_table: np.ndarray, entry_begin: np.ndarray, entry_end: np.ndarray,
                rope_base: float, threads: int | None = None) -> None:
    """oracle_merge_level: one level of the dyadic merge, in place, over
    entries [entry_begin[b], entry_end[b]) of every sequence b."""
    L = lib()
    table = np.ascontiguousarray(page_table, dtype=np.int32)
    eb = np.ascontiguousarray(entry_begin, dtype=np.int32)
    ee = np.ascontiguousarray(entry_end, dtype=np.int32)
    B = table.shape[0]
    rcs = []

    def run(rng):
        rcs.append(L.oracle_merge_level(DT[cache.store], cache.H_kv, cache.d, _p(cache.k), _p(cache.v),
                                        _p(cache.ab), _p(cache.meta), _p(cache.s2), cache.num_pages, _p(table),
                                        table.shape[1], _p(eb), _p(ee), B, float(rope_base), rng[0], rng[1]))

    chunks = _chunks(B, threads or default_threads())
    if len(chunks) == 1:
        run(chunks[0])
    else:
        with ThreadPoolExecutor(len(chunks)) as ex:
            list(ex.map(run, chunks))
    if any(rc != 0 for rc in rcs):
        raise ValueError(f"oracle_merge_level failed: codes {sorted(set(rcs))}")


def compact_range(cache: Cache, page_table: np.ndarray, entry_begin: np.ndarray, lengths: np.ndarray,
                  threads: int | None = None) -> np.ndarray:
    """oracle_compact_range: per sequence and head, the non-null entries of
    [entry_begin[b], lengths[b]) move in order to the front of the range, in
    place; returns the new lengths (int32 [B])."""
    L = lib()
    table = np.ascontiguousarray(page_table, dtype=np.int32)
    eb = np.ascontiguousarray(entry_begin, dtype=np.int32)
    ln = np.ascontiguousarray(lengths, dtype=np.int32)
    B = table.shape[0]
    out = ln.copy()
    rcs = []

    def run(rng):
        rcs.append(L.oracle_compact_range(DT[cache.store], cache.H_kv, cache.d, _p(cache.k), _p(cache.v),
                                          _p(cache.ab), _p(cache.meta), _p(cache.s2), cache.num_pages, _p(table),
                                          table.shape[1], _p(eb), _p(ln), B, _p(out), rng[0], rng[1]))

    chunks = _chunks(B, threads or default_threads())
    if len(chunks) == 1:
        run(chunks[0])
    else:
        with ThreadPoolExecutor(len(chunks)) as ex:
            list(ex.map(run, chunks))
    if any(rc != 0 for rc in rcs):
        raise ValueError(f"oracle_compact_range failed: codes {sorted(set(rcs))}")
    return out


def bf16_round(x: float) -> int:
    return int(lib().oracle_bf16_round(float(x)))


def bf16_value(bits: int) -> float:
    return float(lib().oracle_bf16_value(int(bits)))


def rope(x: np.ndarray, pos: float, base: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib().oracle_rope(_p(y), _p(x), int(x.shape[0]), float(pos), float(base))
    return y


# ---------------------------------------------------------------------------
# per-step policy (equal-variation segments, key-norm landmarks)
# ---------------------------------------------------------------------------

def fix16(bits: int) -> int:
    """bf16 value x -> x * 2^16 rounded half to even, clamped to +-2^28."""
    return int(lib().oracle_fix16(int(bits) & 0xFFFF))


def isqrt_u128(x: int) -> int:
    """floor(sqrt(x)) for 0 <= x < 2^128, as the policy computes it."""
    return int(lib().oracle_isqrt_u128((x >> 64) & 0xFFFFFFFFFFFFFFFF, x & 0xFFFFFFFFFFFFFFFF))


class PolicyResult:
    def __init__(self, seg_offsets, seq_seg_ptr, mask, variation, norm2):
        self.seg_offsets, self.seq_seg_ptr, self.mask = seg_offsets, seq_seg_ptr, mask
        self.variation, self.norm2 = variation, norm2


def policy(k: np.ndarray, v: np.ndarray, seq_offsets: np.ndarray, proj_ptr: np.ndarray,
           proj_idx: np.ndarray, n_segments: int, n_landmarks: int, sink: int, recent: int) -> PolicyResult:
    """oracle_policy: k, v [total_tokens, H, d] bf16 bits (uint16).  Returns the
    N-slot segment offsets [B*N + 1], seq_seg_ptr [B + 1], the protection mask
    [total_tokens, H] and the per-token variation d_t and key norms^2."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    T, H, d = k.shape
    so = np.ascontiguousarray(seq_offsets, dtype=np.int32)
    B = so.shape[0] - 1
    pp = np.ascontiguousarray(proj_ptr, dtype=np.int32)
    pi = np.ascontiguousarray(proj_idx, dtype=np.int32)
    seg = np.zeros(B * n_segments + 1, dtype=np.int32)
    ssp = np.zeros(B + 1, dtype=np.int32)
    mask = np.zeros((T, H), dtype=np.uint8)
    var = np.zeros(T, dtype=np.int64)
    n2 = np.zeros((T, H), dtype=np.uint64)
    rc = lib().oracle_policy(H, d, _p(k), _p(v), _p(so), B, _p(pp), _p(pi) if pi.size else _p(np.zeros(1, np.int32)),
                             pp.shape[0] - 1, n_segments, n_landmarks, sink, recent,
                             _p(seg), _p(ssp), _p(mask), _p(var), _p(n2))
    if rc != 0:
        raise RuntimeError(f"oracle_policy failed ({rc})")
    return PolicyResult(seg, ssp, mask, var, n2)

