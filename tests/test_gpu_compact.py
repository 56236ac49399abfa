"""GPU parity of spicy_compact_range against the oracle's compaction, through
the C ABI.

Compaction moves bytes, so the bar is bit-exactness: every byte of every pool
(keys, values, (alpha, beta), metadata, the variance sidecar) and every new
length equal the oracle's, on the same seeded input.  Inputs: caches of
random contents whose nulls (alpha = -inf) are punched per head at random,
over permuted page tables, with ranges that start mid-page, span several
512-entry rounds, or are empty, all-null or null-free; one range long enough
that its page ids do not all fit the kernel's LDS cache.  Then the real use:
a GPU merge level, GPU compaction, and the decode of the compacted cache
against the oracle's decode of the merged, uncompacted one.
"""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import DEV, _need_gpu, compare_decode, host

pytestmark = pytest.mark.gpu

PAGE = 16
NEG_INF = {"bf16": 0xFF80, "f32": -np.inf}


def random_cache(rng, store, P, H, d, meta=True, diag=False):
    c = oracle.Cache(store, P, H, d, diag=diag)
    for a in (c.k, c.v, c.ab) + ((c.s2,) if diag else ()):
        x = rng.standard_normal(a.shape).astype(np.float32)
        a[:] = (x.view(np.uint32) >> 16).astype(np.uint16) if store == "bf16" else x       # any bits will do
    c.meta["kind"] = rng.integers(1, 3, c.meta.shape)
    c.meta["mass"] = rng.integers(1, 1000, c.meta.shape)
    c.meta["pos_sum"] = rng.integers(0, 1 << 40, c.meta.shape)
    if not meta:
        c.meta = None
    return c


def punch(c, table, b, e0, L, rate, rng):
    """alpha = -inf at a random `rate` of the entries of [e0, L), per head."""
    for e in range(e0, L):
        P, s = table[b, e // PAGE], e % PAGE
        for h in range(c.H_kv):
            if rng.random() < rate[h]:
                c.ab[P, h, s, 0] = NEG_INF[c.store]


def to_gpu(c):
    import coarse_grained_decode_amd as cgd

    def t(a):
        if a is None:
            return None
        if c.store == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    meta = None
    if c.meta is not None:
        meta = torch.from_numpy(np.ascontiguousarray(c.meta).view(np.int32).reshape(c.meta.shape + (4,))).to(DEV)
    return cgd.PagedCache(t(c.k), t(c.v), t(c.ab), meta, t(c.s2))


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def gpu_compact(g, table, begin, lengths):
    import coarse_grained_decode_amd as cgd
    out = torch.full((len(begin),), -7, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    cgd.spicy_compact_range(g, i32(table), i32(begin), i32(lengths), out, err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.item())


def assert_same_pools(g, c):
    for name in ("k", "v", "ab", "s2"):
        ref = getattr(c, name)
        if ref is None:
            continue
        got = host(getattr(g, name))
        assert got.tobytes() == ref.tobytes(), f"{name} differs at {np.argwhere(got != ref)[:5].tolist()}"
    if c.meta is not None:
        got = host(g.meta)
        assert got.tobytes() == np.ascontiguousarray(c.meta).view(np.int32).reshape(got.shape).tobytes(), "meta"


CASES = [
    # (seed, store, H, d, B, max pages, meta, diag, null rates per head)
    (1, "bf16", 4, 128, 6, 110, True, False, (0.5, 0.3, 0.7, 0.0)),
    (2, "f32", 2, 64, 5, 80, True, True, (0.4, 0.9)),
    (3, "bf16", 8, 64, 3, 70, False, False, (0.5,) * 8),
    (4, "f32", 4, 128, 4, 60, True, False, (1.0, 0.2, 0.5, 0.5)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[1]}_H{c[2]}_d{c[3]}" + ("_meta" if c[6] else "") +
                                             ("_diag" if c[7] else "") for c in CASES])
def test_compaction_is_bit_exact(case):
    _need_gpu()
    seed, store, H, d, B, mp, meta, diag, rate = case
    print(f"[compact] case {case}", flush=True)
    rng = np.random.default_rng(seed)
    table = rng.permutation(B * mp + 3).astype(np.int32)[:B * mp].reshape(B, mp)
    c = random_cache(rng, store, B * mp + 3, H, d, meta, diag)
    lengths = rng.integers(1, mp * PAGE + 1, size=B).astype(np.int32)
    lengths[0] = mp * PAGE                                   # several rounds, every page
    begin = (rng.random(B) * lengths).astype(np.int32)
    begin[0] = 13                                            # mid-page
    begin[-1] = lengths[-1]                                  # an empty range
    for b in range(B):
        punch(c, table, b, int(begin[b]), int(lengths[b]), rate, rng)
    if B > 2:                                                # a null-free range
        for e in range(int(begin[1]), int(lengths[1])):
            P, s = table[1, e // PAGE], e % PAGE
            c.ab[P, :, s, 0] = 0
    g = to_gpu(c)
    out, err = gpu_compact(g, table, begin, lengths)
    want = oracle.compact_range(c, table, begin, lengths)
    assert err == 0
    np.testing.assert_array_equal(out, want)
    assert_same_pools(g, c)


def test_long_range_beyond_the_page_cache():
    """One range of 17000 entries (1063 pages: more page ids than the
    kernel keeps in LDS) and a short one."""
    _need_gpu()
    rng = np.random.default_rng(9)
    mp = 1070
    table = rng.permutation(2 * mp).astype(np.int32).reshape(2, mp)
    c = random_cache(rng, "bf16", 2 * mp, 2, 64)
    begin = np.array([5, 30], np.int32)
    lengths = np.array([17005, 400], np.int32)
    for b in range(2):
        punch(c, table, b, int(begin[b]), int(lengths[b]), (0.5, 0.25), rng)
    g = to_gpu(c)
    out, err = gpu_compact(g, table, begin, lengths)
    want = oracle.compact_range(c, table, begin, lengths)
    assert err == 0
    np.testing.assert_array_equal(out, want)
    assert_same_pools(g, c)


def test_bad_ranges_and_pages_leave_sequences_untouched():
    import coarse_grained_decode_amd as cgd
    _need_gpu()
    rng = np.random.default_rng(5)
    mp = 8
    table = np.arange(3 * mp, dtype=np.int32).reshape(3, mp)
    c = random_cache(rng, "bf16", 3 * mp, 2, 64)
    begin = np.array([10, 50, 0], np.int32)
    lengths = np.array([100, 40, 90], np.int32)          # sequence 1: begin past its length
    for b in range(3):
        punch(c, table, b, min(int(begin[b]), int(lengths[b])), int(lengths[b]), (0.5, 0.5), rng)
    bad = table.copy()
    bad[2, 3] = 3 * mp                                    # sequence 2: a page outside the pool
    g = to_gpu(c)
    out, err = gpu_compact(g, bad, begin, lengths)
    assert err == cgd.DEVERR_SEGMENTS | cgd.DEVERR_PAGE_ID
    assert out[1] == 40 and out[2] == 90
    # sequence 0 compacts as the oracle does; 1 and 2 are untouched
    want = oracle.compact_range(c, table[:1], begin[:1], lengths[:1])
    assert out[0] == want[0]
    assert_same_pools(g, c)


def test_merge_compact_decode():
    """GPU merge level, then GPU compaction: the compaction is bit-exact
    against the oracle's compaction of the GPU's merged bytes, and the
    decode of the compacted GPU cache matches the oracle's decode of the
    oracle-merged, uncompacted cache."""
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd import workloads as W
    from test_gpu_merge import gpu_merge, upload_with_meta
    from test_gpu_parity import gpu_decode
    _need_gpu()
    wl = W.qwen2_7b(B=3, T=6000)
    print(f"[compact] merge + compact + decode on {wl.name} B={wl.B}", flush=True)
    ref = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    lengths = None
    for call in wl.calls:
        lengths = oracle.coarsen(call, ref)
    begin = np.zeros(wl.B, np.int32)
    g = upload_with_meta(ref)
    gpu_merge(g, wl, begin, lengths)
    oracle.merge_level(ref, wl.page_table, begin, lengths, wl.calls[-1].rope_base)
    ro, rlse = oracle.decode(wl.q, wl.dtype, ref, wl.H_q, wl.page_table, lengths)
    # the oracle's compaction of the GPU's own merged bytes
    mine = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d, fill=False)
    mine.k[:], mine.v[:], mine.ab[:] = host(g.k), host(g.v), host(g.ab)
    mine.meta[:] = host(g.meta).reshape(-1).view(oracle.META_DTYPE).reshape(mine.meta.shape)
    out, err = gpu_compact(g, wl.page_table, begin, lengths)
    want = oracle.compact_range(mine, wl.page_table, begin, lengths)
    assert err == 0
    np.testing.assert_array_equal(out, want)
    assert (out < lengths).all()
    assert_same_pools(g, mine)
    o, lse = gpu_decode(g, wl, out)
    compare_decode(o, lse, ro, rlse, wl.dtype)
    print(f"[compact] lengths {lengths.tolist()} -> {out.tolist()}", flush=True)
