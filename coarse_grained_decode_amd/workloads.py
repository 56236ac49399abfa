"""Seeded synthetic workloads for SPICY-KV coarsen + decode.

This module builds the inputs both the GPU library and the CPU oracle consume:
keys, values and queries, the protected-token mask, the segment partition, the
page tables and the entry offsets.  It holds none of the method's arithmetic
(no means, variances, rotations, logits or softmax): those live, separately,
in the GPU kernels and in the oracle.

What the generator decides is the cache *policy*, which the pages leave to the
caller of the coarsening step:

* sink and recent tokens stay exact (SPICY-KV demo page, section 1: its
  configuration protects 8 sink and 48 recent tokens);
* "landmark" tokens stay exact (SPICY-KV demo page, Claim 2: C-points); we pick
  the top fraction of tokens by key norm per (sequence, KV head);
* segments: a fixed grid, a two-level dyadic grid sized to hit the target
  compression ratio (SPICY-KV title: dyadic renormalization; Claim 1 (c): the
  coarsening at one or several resolution scales), or equal-variation boundaries (Equal-Variation KV Cache
  page, implementation notes: the total variation is cut into N equal shares,
  and each segment ends where the running variation reaches its share).

Seeds: workload ``c`` draws from ``numpy.random.Generator(PCG64(SeedSequence(1000 + c)))``
children, one child stream per role.  Data are drawn in float32 and, for bf16
workloads, rounded to bfloat16 (ties to even); those bf16 tensors are the inputs
of both paths.  bf16 arrays are carried as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

PAGE = 16
SINK = 8
RECENT = 48
KEY_NOISE = 0.3


# ---------------------------------------------------------------------------
# small helpers (input preparation only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 data to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of stored input data in float64 (bf16 bits are decoded)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


# ---------------------------------------------------------------------------
# containers
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class CoarsenCall:
    """Arguments of one spicy_coarsen call (host copies)."""
    dtype: str                 # "f32" | "bf16"
    H_kv: int
    d: int
    rope_base: float
    k: np.ndarray              # [sum_T, H_kv, d] float32 or uint16 (bf16 bits), pre-RoPE
    v: np.ndarray              # [sum_T, H_kv, d]
    seq_offsets: np.ndarray    # int32 [B+1]
    pos_base: np.ndarray       # int32 [B]
    seg_offsets: np.ndarray    # int32 [n_seg+1]
    seq_seg_ptr: np.ndarray    # int32 [B+1]
    mask: np.ndarray           # uint8 [sum_T, H_kv], 1 = protected (C-point)
    page_table: np.ndarray     # int32 [B, max_pages]
    entry_start: np.ndarray    # int32 [B]

    @property
    def B(self) -> int:
        return int(self.seq_offsets.shape[0] - 1)

    @property
    def n_seg(self) -> int:
        return int(self.seg_offsets.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.seq_offsets[-1])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


@dataclasses.dataclass
class PolicySpec:
    """Inputs of spicy_policy for a per-step chunk: the projection P of the
    equal-variation feature as signed column lists (row r: proj_idx[proj_ptr[r]
    : proj_ptr[r+1]], entry c + 1 for +1 at column c, -(c + 1) for -1), the
    segment slots N per sequence and the landmark rule."""
    proj_ptr: np.ndarray       # int32 [R+1]
    proj_idx: np.ndarray       # int32 [nnz]
    n_segments: int
    n_landmarks: int
    sink: int
    recent: int


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    B: int
    H_q: int
    H_kv: int
    d: int
    rope_base: float
    num_pages: int
    setup: List[CoarsenCall]          # coarsen calls run once, in order
    step: Optional[CoarsenCall]       # coarsen call repeated every step (or None)
    page_table: np.ndarray            # int32 [B, max_pages] used by decode
    q: np.ndarray                     # [B, H_q, d]
    description: str = ""
    shared_prefix_pages: int = 0      # leading logical pages identical in every table row
    policy: Optional[PolicySpec] = None   # device-side policy for the per-step chunk, if offered

    @property
    def calls(self) -> List[CoarsenCall]:
        return self.setup + ([self.step] if self.step is not None else [])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


# ---------------------------------------------------------------------------
# data
# ---------------------------------------------------------------------------

def _run_ids(rng: np.random.Generator, T: int, run: Optional[int], mean_run: Optional[float]) -> np.ndarray:
    """Cluster id per token: fixed runs of `run` tokens, or geometric run lengths."""
    if run is not None:
        return np.arange(T, dtype=np.int64) // run
    lens = rng.geometric(1.0 / mean_run, size=max(16, int(2 * T / mean_run) + 16))
    while lens.sum() < T:
        lens = np.concatenate([lens, rng.geometric(1.0 / mean_run, size=lens.size)])
    return np.repeat(np.arange(lens.size, dtype=np.int64), lens)[:T]


def clustered_keys(rngs, T: int, H: int, d: int, run: Optional[int], mean_run: Optional[float]) -> np.ndarray:
    """Pre-RoPE keys: per KV head a cluster centre ~ N(0, I) per run of tokens,
    plus N(0, 0.3^2 I) noise.  Run boundaries are shared by the heads of a
    sequence; centres are independent per head."""
    rid = _run_ids(rngs["runs"], T, run, mean_run)
    n_runs = int(rid[-1]) + 1 if T else 0
    centres = rngs["centres"].standard_normal((n_runs, H, d), dtype=np.float32)
    keys = centres[rid]
    keys += np.float32(KEY_NOISE) * rngs["noise"].standard_normal((T, H, d), dtype=np.float32)
    return keys


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


# ---------------------------------------------------------------------------
# policy: protection
# ---------------------------------------------------------------------------

def landmark_count(T: int, frac: float) -> int:
    return int(np.floor(frac * T + 0.5))


def protection_mask(k_f64: np.ndarray, sink: int, recent: int, frac: float) -> np.ndarray:
    """mask[t, h] = 1 for the first `sink` tokens, the last `recent` tokens and,
    per KV head, the floor(frac*T + 0.5) largest-norm keys among the others
    (ties go to the lower position).  k_f64: [T, H, d] float64."""
    T, H, _ = k_f64.shape
    mask = np.zeros((T, H), dtype=np.uint8)
    mask[: min(sink, T)] = 1
    if recent > 0:
        mask[max(0, T - recent):] = 1
    L = landmark_count(T, frac)
    if L > 0:
        cand = np.arange(min(sink, T), max(min(sink, T), T - recent))
        norms = np.sqrt(np.einsum("thd,thd->th", k_f64, k_f64))
        for h in range(H):
            nh = norms[cand, h]
            order = np.lexsort((cand, -nh))
            mask[cand[order[:L]], h] = 1
    return mask


# ---------------------------------------------------------------------------
# policy: segmentation (offsets are relative to the sequence start)
# ---------------------------------------------------------------------------

def fixed_segments(T: int, size: int) -> np.ndarray:
    return np.unique(np.concatenate([np.arange(0, T, size), [T]])).astype(np.int64)


def dyadic_plan(T: int, ratio: float, n_protected: int, recent: int = RECENT):
    """Two-level aligned power-of-two grid.

    With cell size s = 2^k, c = ceil(T/s) cells and f cells lying wholly in the
    recent window, n_big = c - (M + f) segments of 2s come first (the oldest
    tokens, aligned from position 0) and n_small = 2(M + f) - c segments of s
    follow (the last one cut at T), where M = round(T/ratio) - n_protected is
    the number of macro-nodes wanted.  The smallest k with n_big >= 0 and
    n_small >= f + 1 is taken.  Returns (s, n_big, n_small)."""
    M = int(round(T / ratio)) - n_protected
    if M <= 0:
        raise ValueError("compression ratio leaves no macro-nodes")
    k = 0
    while (1 << k) <= 2 * T:
        s = 1 << k
        c = -(-T // s)
        f = sum(1 for j in range(c) if j * s >= T - recent)
        n_big = c - (M + f)
        n_small = 2 * (M + f) - c
        if n_big >= 0 and n_small >= f + 1:
            return s, n_big, n_small
        k += 1
    raise ValueError("no dyadic grid fits")


def dyadic_segments(T: int, ratio: float, n_protected: int) -> np.ndarray:
    s, n_big, n_small = dyadic_plan(T, ratio, n_protected)
    bounds = [0]
    for _ in range(n_big):
        bounds.append(bounds[-1] + 2 * s)
    for _ in range(n_small):
        bounds.append(min(T, bounds[-1] + s))
    bounds[-1] = T
    b = np.asarray(bounds, dtype=np.int64)
    assert np.all(np.diff(b) > 0)
    return b


def variation_quanta(k_f64: np.ndarray, v_f64: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """Quantised local variation d_t of the projected key/value trajectory
    z_t = P [k_t; v_t] (all KV heads concatenated): d_0 = 0,
    d_t = ||z_t - z_{t-1}||_2, stored as round(d_t * 2^32) in int64 so that
    the cumulative sum and the threshold search below are exact integers."""
    T = k_f64.shape[0]
    x = np.concatenate([k_f64.reshape(T, -1), v_f64.reshape(T, -1)], axis=1)
    z = x @ proj.T
    dz = np.zeros(T, dtype=np.float64)
    if T > 1:
        dz[1:] = np.sqrt(np.sum((z[1:] - z[:-1]) ** 2, axis=1))
    return np.rint(dz * 4294967296.0).astype(np.int64)


def equal_variation_segments(quanta: np.ndarray, N: int) -> np.ndarray:
    """Equal-variation boundaries (Equal-Variation KV Cache page, "Mathematical
    statement" and "Implementation notes"): with the cumulative variation
    C_t = sum_{r<=t} d_r and thresholds Q_j = floor(j C_last / N), j = 1..N-1,
    boundary b_j = min{t : C_t >= Q_j} (first hitting time); the crossing token
    starts the new segment; empty segments are dropped."""
    T = quanta.shape[0]
    C = np.cumsum(quanta)
    total = int(C[-1]) if T else 0
    bounds = [0]
    for j in range(1, N):
        Q = (j * total) // N
        b = int(np.searchsorted(C, Q, side="left"))
        bounds.append(min(b, T))
    bounds.append(T)
    return np.unique(np.asarray(bounds, dtype=np.int64))


def sparse_sign_projection(rng: np.random.Generator, rows: int, cols: int,
                           density: float) -> Tuple[np.ndarray, np.ndarray]:
    """A very sparse random projection (Li, Hastie and Church, 2006): each
    entry is +1 or -1 with probability density/2 and 0 otherwise, drawn row
    by row.  Returned as (proj_ptr [rows+1], proj_idx [nnz]) with signed
    1-based column ids; a row that draws no entry gets one random +-1 so that
    every feature sees the input."""
    ptr, idx = [0], []
    for _ in range(rows):
        u = rng.random(cols)
        cols_r = np.nonzero(u < density)[0]
        if cols_r.size == 0:
            cols_r = rng.integers(0, cols, size=1)
        sign = np.where(rng.random(cols_r.size) < 0.5, 1, -1)
        idx.extend((sign * (cols_r + 1)).tolist())
        ptr.append(len(idx))
    return np.asarray(ptr, dtype=np.int32), np.asarray(idx, dtype=np.int32)


def policy_spec(rng: np.random.Generator, H: int, d: int, n_segments: int, n_landmarks: int,
                sink: int = 0, recent: int = 0, rows: int = 16) -> PolicySpec:
    """Policy inputs with a 16-row projection of [k; v] at density 1/sqrt(2 H d)."""
    D = 2 * H * d
    ptr, idx = sparse_sign_projection(rng, rows, D, 1.0 / np.sqrt(D))
    return PolicySpec(ptr, idx, n_segments, n_landmarks, sink, recent)


# ---------------------------------------------------------------------------
# assembling coarsen calls
# ---------------------------------------------------------------------------

def _concat_call(dtype, H, d, base, ks, vs, masks, segs, pos_base, page_table, entry_start) -> CoarsenCall:
    B = len(ks)
    Ts = [k.shape[0] for k in ks]
    seq_offsets = np.zeros(B + 1, dtype=np.int64)
    seq_offsets[1:] = np.cumsum(Ts)
    seg_off = [np.zeros(1, dtype=np.int64)]
    seq_seg_ptr = np.zeros(B + 1, dtype=np.int64)
    for b in range(B):
        sb = segs[b]
        assert sb[0] == 0 and sb[-1] == Ts[b]
        seg_off.append(sb[1:] + seq_offsets[b])
        seq_seg_ptr[b + 1] = seq_seg_ptr[b] + (len(sb) - 1)
    seg_offsets = np.concatenate(seg_off)
    k = np.concatenate(ks, axis=0) if B else np.zeros((0, H, d), ks[0].dtype if ks else np.float32)
    v = np.concatenate(vs, axis=0) if B else np.zeros_like(k)
    return CoarsenCall(
        dtype=dtype, H_kv=H, d=d, rope_base=float(base),
        k=np.ascontiguousarray(k), v=np.ascontiguousarray(v),
        seq_offsets=seq_offsets.astype(np.int32),
        pos_base=np.asarray(pos_base, dtype=np.int32),
        seg_offsets=seg_offsets.astype(np.int32),
        seq_seg_ptr=seq_seg_ptr.astype(np.int32),
        mask=np.ascontiguousarray(np.concatenate(masks, axis=0)).astype(np.uint8),
        page_table=np.ascontiguousarray(page_table, dtype=np.int32),
        entry_start=np.asarray(entry_start, dtype=np.int32),
    )


def entry_bound(segs: np.ndarray, mask: np.ndarray) -> int:
    """Upper bound on entries per (sequence, head): one macro-node per segment
    plus every protected token.  Used only to size page tables."""
    return int(len(segs) - 1 + mask.sum(axis=0).max(initial=0))


def _rngs(config_id: int) -> dict:
    names = ["centres", "noise", "values", "queries", "runs", "ctx", "perm", "proj", "suffix"]
    children = np.random.SeedSequence(1000 + config_id).spawn(len(names))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(names, children)}


def _sequence(rngs, T, H, d, dtype, run, mean_run, frac, sink, recent):
    kf = clustered_keys(rngs, T, H, d, run, mean_run)
    vf = rngs["values"].standard_normal((T, H, d), dtype=np.float32)
    k = _store(kf, dtype)
    v = _store(vf, dtype)
    mask = protection_mask(as_f64(k, dtype), sink, recent, frac)
    return k, v, mask


def _query(rngs, B, H_q, d, dtype):
    return _store(rngs["queries"].standard_normal((B, H_q, d), dtype=np.float32), dtype)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def make_single(config_id: int, *, dtype: str, B: int, H_q: int, H_kv: int, d: int,
                rope_base: float, T, run: Optional[int], mean_run: Optional[float],
                frac: float, ratio: Optional[float], grid: Optional[int],
                permute: bool, name: str, description: str = "") -> Workload:
    """One coarsen call over B sequences followed by decode.  T is an int or a
    list of per-sequence lengths."""
    rngs = _rngs(config_id)
    Ts = [int(t) for t in (T if np.ndim(T) else [T] * B)]
    ks, vs, masks, segs = [], [], [], []
    for b in range(B):
        k, v, mask = _sequence(rngs, Ts[b], H_kv, d, dtype, run, mean_run, frac, SINK, RECENT)
        n_prot = SINK + RECENT + landmark_count(Ts[b], frac)
        if grid is not None:
            sb = fixed_segments(Ts[b], grid)
        else:
            sb = dyadic_segments(Ts[b], ratio, n_prot)
        ks.append(k); vs.append(v); masks.append(mask); segs.append(sb)
    pages_b = [-(-entry_bound(segs[b], masks[b]) // PAGE) for b in range(B)]
    max_pages = max(pages_b) if B else 1
    num_pages = int(sum(pages_b))
    ids = np.arange(num_pages, dtype=np.int64)
    if permute:
        ids = rngs["perm"].permutation(num_pages)
    table = np.full((B, max_pages), -1, dtype=np.int64)
    pos = 0
    for b in range(B):
        table[b, : pages_b[b]] = ids[pos: pos + pages_b[b]]
        pos += pages_b[b]
    call = _concat_call(dtype, H_kv, d, rope_base, ks, vs, masks, segs,
                        np.zeros(B, dtype=np.int64), table, np.zeros(B, dtype=np.int64))
    q = _query(rngs, B, H_q, d, dtype)
    return Workload(name=name, dtype=dtype, B=B, H_q=H_q, H_kv=H_kv, d=d, rope_base=rope_base,
                    num_pages=num_pages, setup=[call], step=None,
                    page_table=call.page_table, q=q, description=description)


def make_shared_prefix(config_id: int = 4, *, B: int = 32, H_q: int = 28, H_kv: int = 4, d: int = 128,
                       prefix_T: int = 65536, suffix_range=(512, 2048), chunk_T: int = 8192,
                       ratio: float = 28.6, frac: float = 0.01, mean_run: float = 48.0,
                       rope_base: float = 1e6, name: str = "shared_prefix") -> Workload:
    """Shared compressed prefix + private exact suffix + a fresh chunk coarsened
    with equal-variation segments every step.

    Positions: prefix [0, prefix_T), suffix [prefix_T, prefix_T + S_b), chunk
    after the suffix.  Logical pages of sequence b: the shared prefix pages
    (null-padded to a page boundary) | the suffix's exact entries | the chunk's
    entries.  All page tables point at the same physical prefix pages."""
    dtype = "bf16"
    rngs = _rngs(config_id)
    # prefix: one sequence, dyadic segments at the target ratio
    kp, vp, mp = _sequence(rngs, prefix_T, H_kv, d, dtype, None, mean_run, frac, SINK, RECENT)
    sp = dyadic_segments(prefix_T, ratio, SINK + RECENT + landmark_count(prefix_T, frac))
    prefix_pages = -(-entry_bound(sp, mp) // PAGE)
    # suffixes: exact tokens (all protected, one segment each)
    S = rngs["suffix"].integers(suffix_range[0], suffix_range[1] + 1, size=B)
    # chunk: equal-variation segments; protection = landmarks only
    n_land = landmark_count(chunk_T, frac)
    N = int(round(chunk_T / ratio)) - n_land
    chunk_pages = -(-(N + n_land) // PAGE)
    suffix_pages = [-(-int(s) // PAGE) for s in S]
    max_pages = prefix_pages + max(suffix_pages) + chunk_pages
    num_pages = prefix_pages + int(sum(suffix_pages)) + B * chunk_pages
    table = np.full((B, max_pages), -1, dtype=np.int64)
    nxt = prefix_pages
    for b in range(B):
        table[b, :prefix_pages] = np.arange(prefix_pages)
        table[b, prefix_pages: prefix_pages + suffix_pages[b]] = np.arange(nxt, nxt + suffix_pages[b])
        nxt += suffix_pages[b]
        c0 = prefix_pages + suffix_pages[b]
        table[b, c0: c0 + chunk_pages] = np.arange(nxt, nxt + chunk_pages)
        nxt += chunk_pages
    assert nxt == num_pages

    prefix_table = np.arange(prefix_pages, dtype=np.int64)[None, :]
    prefix_call = _concat_call(dtype, H_kv, d, rope_base, [kp], [vp], [mp], [sp], [0],
                               prefix_table, [0])

    ks, vs, ms, ss = [], [], [], []
    for b in range(B):
        T = int(S[b])
        kf = clustered_keys(rngs, T, H_kv, d, None, mean_run)
        vf = rngs["values"].standard_normal((T, H_kv, d), dtype=np.float32)
        ks.append(_store(kf, dtype)); vs.append(_store(vf, dtype))
        ms.append(np.ones((T, H_kv), dtype=np.uint8))
        ss.append(np.asarray([0, T], dtype=np.int64))
    suffix_call = _concat_call(dtype, H_kv, d, rope_base, ks, vs, ms, ss,
                               np.full(B, prefix_T), table, np.full(B, prefix_pages * PAGE))

    proj = rngs["proj"].standard_normal((16, 2 * H_kv * d))
    ks, vs, ms, ss = [], [], [], []
    for b in range(B):
        k, v, mask = _sequence(rngs, chunk_T, H_kv, d, dtype, None, mean_run, frac, 0, 0)
        seg = equal_variation_segments(variation_quanta(as_f64(k, dtype), as_f64(v, dtype), proj), N)
        ks.append(k); vs.append(v); ms.append(mask); ss.append(seg)
    entry_start = [(prefix_pages + suffix_pages[b]) * PAGE for b in range(B)]
    chunk_call = _concat_call(dtype, H_kv, d, rope_base, ks, vs, ms, ss,
                              prefix_T + S, table, entry_start)
    q = _query(rngs, B, H_q, d, dtype)
    pol = policy_spec(np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + config_id, 7]))),
                      H_kv, d, N, n_land)
    return Workload(name=name, dtype=dtype, B=B, H_q=H_q, H_kv=H_kv, d=d, rope_base=rope_base,
                    num_pages=num_pages, setup=[prefix_call, suffix_call], step=chunk_call,
                    page_table=np.ascontiguousarray(table, dtype=np.int32), q=q,
                    shared_prefix_pages=prefix_pages, policy=pol,
                    description=f"{B} seqs share a {prefix_T}-token prefix at {ratio}x; "
                                f"suffix U[{suffix_range[0]},{suffix_range[1]}] exact; "
                                f"{chunk_T}-token chunk per step, equal-variation N={N}")


def chunked(x: np.ndarray) -> np.ndarray:
    """[P, H, 16, d] entry rows in the cache's page layout [P, H, d/W, 16, W],
    W = min(8, d)."""
    P, H, S, d = x.shape
    W = d if d < 8 else 8
    return np.ascontiguousarray(x.reshape(P, H, S, d // W, W).transpose(0, 1, 3, 2, 4))


@dataclasses.dataclass
class DecodeCase:
    """Cache contents and a batch for decode-only cases (no coarsening):
    k, v [P, H, d/W, 16, W] (the cache's page layout), ab [P, H, 16, 2] in storage format
    (bf16 bits or float32), page_table int32 [B, max_pages], lengths int32 [B],
    q [B, H_q, d]."""
    dtype: str
    H_q: int
    H_kv: int
    d: int
    k: np.ndarray
    v: np.ndarray
    ab: np.ndarray
    page_table: np.ndarray
    lengths: np.ndarray
    q: np.ndarray
    shared_prefix_pages: int


def random_decode_case(seed: int, *, B: int, H_q: int, H_kv: int, d: int, dtype: str = "bf16",
                       prefix_pages: int = 0, private_pages: Tuple[int, int] = (1, 6),
                       null_frac: float = 0.05, q_tokens: int = 1) -> DecodeCase:
    """A synthetic paged cache for decode tests: keys, values and queries
    N(0, 1); alpha ~ U(0, 4) (a null_frac share of entries null: alpha = -inf);
    beta ~ U(0, 0.01).  Every sequence maps the same `prefix_pages` physical
    pages first, then U[private_pages] private pages in a shuffled pool; its
    length ends at a random slot of its last page.  Slots past a sequence's
    length in its own last private page hold NaN, so reading them would show.  With
    q_tokens > 1 the queries are [B, q_tokens, H_q, d]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(5000 + seed)))
    npriv = rng.integers(private_pages[0], private_pages[1] + 1, size=B)
    num_pages = prefix_pages + int(npriv.sum())
    max_pages = prefix_pages + int(npriv.max())
    k = rng.standard_normal((num_pages, H_kv, PAGE, d), dtype=np.float32)
    v = rng.standard_normal((num_pages, H_kv, PAGE, d), dtype=np.float32)
    ab = np.empty((num_pages, H_kv, PAGE, 2), dtype=np.float32)
    ab[..., 0] = rng.uniform(0.0, 4.0, size=ab.shape[:-1])
    ab[..., 0][rng.random(ab.shape[:-1]) < null_frac] = -np.inf
    ab[..., 1] = rng.uniform(0.0, 0.01, size=ab.shape[:-1])
    pool = prefix_pages + rng.permutation(int(npriv.sum()))
    table = np.full((B, max_pages), -1, dtype=np.int32)
    lengths = np.empty(B, dtype=np.int32)
    nxt = 0
    for b in range(B):
        n = int(npriv[b])
        table[b, :prefix_pages] = np.arange(prefix_pages)
        table[b, prefix_pages:prefix_pages + n] = pool[nxt:nxt + n]
        nxt += n
        used = int(rng.integers(1, PAGE + 1))
        lengths[b] = (prefix_pages + n - 1) * PAGE + used
        if n > 0:           # a shared page holds other sequences' entries: leave it whole
            last = table[b, prefix_pages + n - 1]
            k[last, :, used:, :] = np.nan
            v[last, :, used:, :] = np.nan
            ab[last, :, used:, :] = np.nan
    q = rng.standard_normal((B, H_q, d) if q_tokens == 1 else (B, q_tokens, H_q, d), dtype=np.float32)
    return DecodeCase(dtype, H_q, H_kv, d, _store(chunked(k), dtype), _store(chunked(v), dtype),
                      _store(ab, dtype), table, lengths, _store(q, dtype), prefix_pages)


def token_weights(call: "CoarsenCall", seed: int, hi: int = 1 << 20) -> np.ndarray:
    """Per-token integer weights for a coarsen call (int64 [total_tokens]):
    U[0, hi), a fifth of them 0, and every token of every 7th segment 0 (so
    some macro-nodes fall back to the plain mean)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5700 + seed, call.total_tokens])))
    w = rng.integers(0, hi, size=call.total_tokens, dtype=np.int64)
    w[rng.random(call.total_tokens) < 0.2] = 0
    so = np.asarray(call.seg_offsets)
    for s in range(0, len(so) - 1, 7):
        w[so[s]:so[s + 1]] = 0
    return w


def random_variances(c: DecodeCase, seed: int, scale: float = 2.0) -> np.ndarray:
    """Per-dimension variances for a DecodeCase's entries (the diagonal
    closure's sidecar, the cache's k layout, storage format): U(0, scale),
    NaN wherever the case planted NaN (slots past a sequence's length)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5500 + seed, c.d])))
    P, H = c.ab.shape[:2]
    s2 = rng.uniform(0.0, scale, size=(P, H, PAGE, c.d)).astype(np.float32)
    alpha = c.ab[..., 0]
    if c.dtype == "bf16":
        alpha = (alpha.astype(np.uint32) << 16).view(np.float32)
    s2[np.isnan(alpha)] = np.nan
    return _store(chunked(s2), c.dtype)


@dataclasses.dataclass
class PolicyCase:
    """Inputs of one spicy_policy call (host copies, bf16 bits)."""
    k: np.ndarray              # uint16 [sum_T, H, d]
    v: np.ndarray              # uint16 [sum_T, H, d]
    seq_offsets: np.ndarray    # int32 [B+1]
    spec: PolicySpec


def random_policy_case(seed: int, *, B: int, T_range: Tuple[int, int], H: int, d: int, n_segments: int,
                       n_landmarks: int, sink: int = 0, recent: int = 0, mean_run: float = 48.0,
                       proj_rows: int = 16) -> PolicyCase:
    """Clustered keys (geometric runs, as the benchmark workloads) and N(0, 1)
    values for B sequences of U[T_range] tokens, with a seeded very sparse
    projection of [k; v]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(7000 + seed)))
    rngs = {r: np.random.Generator(np.random.PCG64(ss))
            for r, ss in zip(("runs", "centres", "noise", "values"), rng.bit_generator.seed_seq.spawn(4))}
    Ts = rng.integers(T_range[0], T_range[1] + 1, size=B)
    ks, vs = [], []
    for T in Ts:
        ks.append(_store(clustered_keys(rngs, int(T), H, d, None, mean_run), "bf16"))
        vs.append(_store(rngs["values"].standard_normal((int(T), H, d), dtype=np.float32), "bf16"))
    so = np.zeros(B + 1, dtype=np.int32)
    so[1:] = np.cumsum(Ts)
    D = 2 * H * d
    ptr, idx = sparse_sign_projection(rng, proj_rows, D, 1.0 / np.sqrt(D))
    spec = PolicySpec(ptr, idx, n_segments, n_landmarks, sink, recent)
    k = np.concatenate(ks) if B else np.zeros((0, H, d), np.uint16)
    v = np.concatenate(vs) if B else np.zeros((0, H, d), np.uint16)
    return PolicyCase(k, v, so, spec)


def query_tokens(wl: Workload, n_q: int) -> np.ndarray:
    """n_q query tokens per sequence for wl ([B, n_q, H_q, d], N(0, 1) in the
    workload's dtype), from a stream of their own: SeedSequence([2000, n_q])."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2000, n_q])))
    return _store(rng.standard_normal((wl.B, n_q, wl.H_q, wl.d), dtype=np.float32), wl.dtype)


def tiny_fp32(**over) -> Workload:
    """Single-head fp32 case: d=64, T=1024, runs of 32, 16-token grid, base 1e4."""
    kw = dict(dtype="f32", B=1, H_q=1, H_kv=1, d=64, rope_base=1e4, T=1024, run=32,
              mean_run=None, frac=0.01, ratio=None, grid=16, permute=False, name="tiny_fp32",
              description="B1, 1/1 heads, d64, T1024, fp32, 16-token segments")
    kw.update(over)
    return make_single(0, **kw)


def qwen2_1p5b(**over) -> Workload:
    kw = dict(dtype="bf16", B=8, H_q=12, H_kv=2, d=128, rope_base=1e6, T=10752, run=32,
              mean_run=None, frac=0.01, ratio=28.6, grid=None, permute=False, name="qwen2_1.5b_layer",
              description="B8, 12/2 heads, d128, T10752, bf16, dyadic 28.6x")
    kw.update(over)
    return make_single(1, **kw)


def qwen2_7b(**over) -> Workload:
    kw = dict(dtype="bf16", B=16, H_q=28, H_kv=4, d=128, rope_base=1e6, T=32768, run=None,
              mean_run=48.0, frac=0.01, ratio=28.6, grid=None, permute=False, name="qwen2_7b_layer",
              description="B16, 28/4 heads, d128, T32768, bf16, dyadic 28.6x")
    kw.update(over)
    return make_single(2, **kw)


def long_ragged(T_range=(65536, 131072), **over) -> Workload:
    B = over.pop("B", 8)
    rng = _rngs(3)["ctx"]
    Ts = rng.integers(T_range[0], T_range[1] + 1, size=B)
    kw = dict(dtype="bf16", B=B, H_q=28, H_kv=4, d=128, rope_base=1e6, T=list(Ts), run=None,
              mean_run=48.0, frac=0.005, ratio=50.0, grid=None, permute=True, name="long_ragged",
              description=f"B{B}, 28/4 heads, T~U[{T_range[0]},{T_range[1]}], bf16, dyadic 50x, permuted pages")
    kw.update(over)
    return make_single(3, **kw)


def shared_prefix(**over) -> Workload:
    return make_shared_prefix(4, **over)


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "qwen2_1.5b_layer": qwen2_1p5b,
    "qwen2_7b_layer": qwen2_7b,
    "long_ragged": long_ragged,
    "shared_prefix": shared_prefix,
}
