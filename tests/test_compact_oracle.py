"""Pins of the oracle's compaction of a merged range (oracle_compact_range)
against things other than itself.

SPICY-KV demo page, Claim 12 (the cascaded dyadic ring-buffer pyramid): once
a level has merged, half of its slots hold nulls; compaction gives them back.
Per sequence and KV head the non-null entries (alpha != -inf) of
[entry_begin, length) move, in order, to the front of the range; the new
length is entry_begin plus the longest head's count; the rest of each head up
to the end of the new last page becomes nulls.  Pins:
  * a hand-built cache over a non-identity page table, with the range
    crossing pages: the expected pools are built here, entry by entry, from
    the documented layout;
  * a freshly coarsened cache is already compact (bytes and lengths equal);
  * after a merge level: every head's non-null entry sequence is unchanged
    byte for byte, the decode is unchanged, the new length and the null tail
    follow the rule, entries before the range and pages past the new last
    page are untouched; compacting again changes nothing;
  * a pyramid that compacts after every merge leaves, entry by entry, the
    cache the coarsening of the joined segments writes directly (the
    coarsening is pinned to numpy on its own);
  * bad ranges and page ids are refused and leave the cache untouched.
"""
import numpy as np
import pytest

import oracle
from coarse_grained_decode_amd import workloads as W
from coarse_grained_decode_amd.runner import DyadicPyramid

PAGE = 16


def snapshot(cache):
    return {n: getattr(cache, n).copy() for n in ("k", "v", "ab", "meta")}


def same_bytes(a, b):
    return all(a[n].tobytes() == b[n].tobytes() for n in a)


def entry(cache, table, b, h, e):
    """Every stored field of logical entry e of sequence b, head h, read with
    the layout k[P, h, i // W, slot, i % W] (W = min(8, d))."""
    P, s = int(table[b, e // PAGE]), e % PAGE
    return (cache.k[P, h, :, s, :].tobytes(), cache.v[P, h, :, s, :].tobytes(),
            cache.ab[P, h, s].tobytes(), cache.meta[P, h, s].tobytes())


def neg_inf(cache, x):
    """alpha == -inf (bfloat16 pools hold the bits: 0xFF80)."""
    return x == 0xFF80 if cache.store == "bf16" else np.isneginf(x)


def is_null(cache, table, b, h, e):
    P, s = int(table[b, e // PAGE]), e % PAGE
    return (neg_inf(cache, cache.ab[P, h, s, 0]) and cache.ab[P, h, s, 1] == 0 and
            not np.any(cache.k[P, h, :, s, :]) and not np.any(cache.v[P, h, :, s, :]) and
            int(cache.meta[P, h, s]["kind"]) == 0 and int(cache.meta[P, h, s]["mass"]) == 0)


def live(cache, table, b, h, e0, e1):
    return [entry(cache, table, b, h, e) for e in range(e0, e1)
            if not neg_inf(cache, cache.ab[int(table[b, e // PAGE]), h, e % PAGE, 0])]


def test_hand_built_cache():
    """Two heads, d = 4 (W = 4), one sequence over pages [5, 0, 3, 1], range
    [13, 42): head 0 keeps 20 entries, head 1 keeps 9; expected pools written
    here from the layout."""
    H, d, npg = 2, 4, 6
    table = np.array([[5, 0, 3, 1]], np.int32)
    c = oracle.Cache("f64", npg, H, d)
    rng = np.random.default_rng(11)
    c.k[:] = rng.standard_normal(c.k.shape)
    c.v[:] = rng.standard_normal(c.v.shape)
    c.ab[:] = rng.standard_normal(c.ab.shape)
    c.meta["kind"] = rng.integers(1, 3, c.meta.shape)
    c.meta["mass"] = rng.integers(1, 50, c.meta.shape)
    c.meta["pos_sum"] = rng.integers(0, 1 << 40, c.meta.shape)
    e0, L = 13, 42
    nulls = {0: {14, 15, 16, 20, 22, 30, 31, 33, 40}, 1: set(range(13, 42)) - {13, 17, 18, 25, 29, 34, 38, 39, 41}}
    for h in range(H):
        for e in nulls[h]:
            P, s = table[0, e // PAGE], e % PAGE
            c.ab[P, h, s, 0] = -np.inf
    before = snapshot(c)
    want = oracle.Cache("f64", npg, H, d)
    for n in ("k", "v", "ab", "meta"):
        getattr(want, n)[:] = before[n]
    keep = {h: [e for e in range(e0, L) if e not in nulls[h]] for h in range(H)}
    new_len = e0 + max(len(keep[h]) for h in range(H))
    assert new_len == 33
    for h in range(H):
        src = [entry(c, table, 0, h, e) for e in keep[h]]
        for i, (kb, vb, ab, mb) in enumerate(src):
            P, s = table[0, (e0 + i) // PAGE], (e0 + i) % PAGE
            want.k[P, h, :, s, :] = np.frombuffer(kb, np.float64).reshape(1, d)
            want.v[P, h, :, s, :] = np.frombuffer(vb, np.float64).reshape(1, d)
            want.ab[P, h, s] = np.frombuffer(ab, np.float64)
            want.meta[P, h, s] = np.frombuffer(mb, oracle.META_DTYPE)[0]
        for e in range(e0 + len(src), 48):                 # to the end of the page of entry 32
            P, s = table[0, e // PAGE], e % PAGE
            want.k[P, h, :, s, :] = 0
            want.v[P, h, :, s, :] = 0
            want.ab[P, h, s] = (-np.inf, 0.0)
            want.meta[P, h, s] = (0, 0, 0)
    out = oracle.compact_range(c, table, np.array([e0]), np.array([L]))
    assert out.tolist() == [new_len]
    assert same_bytes(snapshot(c), snapshot(want))
    # pages 2 and 4 are not the sequence's: untouched (checked above as part
    # of the whole pools); page 1 (entries 48..63) lies past the new last page
    assert c.k[1].tobytes() == before["k"][1].tobytes()


def merge_fixture(seed, B=3, H=2, d=32, n_seg=12, store="f64", base=1e4):
    """Coarsened sequences with a protected 10% (never a segment's first
    token), entries starting at 5 (entries 0..4 hold older data)."""
    rng = np.random.default_rng(seed)
    ks, vs, ms, ss = [], [], [], []
    for b in range(B):
        lens = rng.integers(4, 14, size=n_seg)
        T = int(lens.sum())
        segs = np.concatenate([[0], np.cumsum(lens)])
        ks.append(rng.standard_normal((T, H, d)) + rng.standard_normal((1, H, d)))
        vs.append(rng.standard_normal((T, H, d)))
        m = rng.random((T, H)) < 0.1
        m[segs[:-1], :] = False
        ms.append(m)
        ss.append(segs)
    mp = 16
    table = rng.permutation(B * mp).astype(np.int32).reshape(B, mp)
    start = np.full(B, 5, np.int32)
    call = W._concat_call("f64", H, d, base, ks, vs, ms, ss, np.full(B, 40), table, start)
    cache = oracle.Cache(store, B * mp, H, d)
    lengths = oracle.coarsen(call, cache, in_dtype="f64")
    return cache, table, start, lengths


@pytest.mark.parametrize("store", ["f64", "bf16", "f32"])
def test_fresh_coarsening_is_already_compact(store):
    cache, table, start, lengths = merge_fixture(2, store=store)
    before = snapshot(cache)
    out = oracle.compact_range(cache, table, start, lengths)
    np.testing.assert_array_equal(out, lengths)
    assert same_bytes(before, snapshot(cache))


@pytest.mark.parametrize("store", ["f64", "bf16"])
def test_after_a_merge(store):
    cache, table, start, lengths = merge_fixture(3, store=store)
    B, H = table.shape[0], cache.H_kv
    oracle.merge_level(cache, table, start, lengths, 1e4)
    before = snapshot(cache)
    q = np.random.default_rng(4).standard_normal((B, 4 * H, cache.d))
    o1, l1 = oracle.decode(q, "f64", cache, 4 * H, table, lengths)
    lives = {(b, h): live(cache, table, b, h, int(start[b]), int(lengths[b])) for b in range(B) for h in range(H)}
    out = oracle.compact_range(cache, table, start, lengths)
    after = snapshot(cache)
    for b in range(B):
        e0 = int(start[b])
        counts = [len(lives[b, h]) for h in range(H)]
        assert out[b] == e0 + max(counts) < lengths[b]
        pad_end = -(-int(out[b]) // PAGE) * PAGE
        for h in range(H):
            got = [entry(cache, table, b, h, e) for e in range(e0, e0 + counts[h])]
            assert got == lives[b, h]
            assert all(is_null(cache, table, b, h, e) for e in range(e0 + counts[h], pad_end))
            for e in range(e0):
                P, s = table[b, e // PAGE], e % PAGE
                assert cache.ab[P, h, s].tobytes() == before["ab"][P, h, s].tobytes()
                assert cache.k[P, h, :, s].tobytes() == before["k"][P, h, :, s].tobytes()
        for lp in range(pad_end // PAGE, table.shape[1]):             # freed and unused pages untouched
            P = table[b, lp]
            for n in after:
                assert after[n][P].tobytes() == before[n][P].tobytes()
    o2, l2 = oracle.decode(q, "f64", cache, 4 * H, table, out)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)
    again = oracle.compact_range(cache, table, start, out)
    np.testing.assert_array_equal(again, out)
    assert same_bytes(after, snapshot(cache))


def test_empty_and_all_null_ranges():
    cache, table, start, lengths = merge_fixture(5, B=2)
    H = cache.H_kv
    # sequence 0: an empty range at its end; sequence 1: every entry of the
    # range turned null
    b = 1
    for e in range(int(start[b]), int(lengths[b])):
        P, s = table[b, e // PAGE], e % PAGE
        cache.ab[P, :, s, 0] = -np.inf
    eb = np.array([lengths[0], start[1]], np.int32)
    out = oracle.compact_range(cache, table, eb, lengths)
    assert out.tolist() == [int(lengths[0]), int(start[1])]
    for h in range(H):
        assert all(is_null(cache, table, 1, h, e) for e in range(int(start[1]), PAGE))


def test_refusals_leave_the_cache_untouched():
    cache, table, start, lengths = merge_fixture(6, B=2)
    before = snapshot(cache)
    with pytest.raises(ValueError, match="codes"):
        oracle.compact_range(cache, table, lengths + 1, lengths)          # begin past the length
    bad = table.copy()
    bad[1, 1] = cache.num_pages                                         # a page outside the pool
    with pytest.raises(ValueError, match="codes"):
        oracle.compact_range(cache, bad, np.zeros(2, np.int32), lengths, threads=1)
    with pytest.raises(ValueError, match="codes"):                      # beyond the table's pages
        oracle.compact_range(cache, table[:, :1], np.zeros(2, np.int32), lengths)
    # sequence 0 came before the bad one in the single-threaded run: it was
    # compacted (it had nothing to move); sequence 1 is untouched
    assert same_bytes(before, snapshot(cache))


@pytest.mark.parametrize("base", [1e4, 0.0])
def test_compacting_pyramid_is_the_coarsening_of_joined_segments(base):
    """Four chunks of four segments, appended at the current length, merged
    by the dyadic schedule and compacted after every merge: every entry,
    null or not, at every index of [0, length), and the length itself, are
    those of the coarsening of the same tokens with one segment per chunk."""
    B, H, d, mp = 2, 2, 32, 40
    rng = np.random.default_rng(7)
    data = []
    for c in range(4):
        per = []
        for b in range(B):
            lens = rng.integers(5, 13, size=4)
            T = int(lens.sum())
            segs = np.concatenate([[0], np.cumsum(lens)])
            k = rng.standard_normal((T, H, d)) + rng.standard_normal((1, H, d))
            m = rng.random((T, H)) < 0.1
            m[segs[:-1], :] = False
            per.append((k, rng.standard_normal((T, H, d)), m, segs))
        data.append(per)
    table = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
    cache = oracle.Cache("f64", B * mp, H, d)
    lengths = np.zeros(B, np.int32)
    pos = np.full(B, 100, np.int64)
    pyr = DyadicPyramid(B)
    peak = 0
    for per in data:
        call = W._concat_call("f64", H, d, base, [x[0] for x in per], [x[1] for x in per], [x[2] for x in per],
                              [x[3] for x in per], pos, table, lengths)
        begin = lengths.copy()
        lengths = oracle.coarsen(call, cache, in_dtype="f64")
        peak = max(peak, int(lengths.max()))
        pyr.push(begin, lengths)
        while (m := pyr.next_merge()) is not None:
            oracle.merge_level(cache, table, m[0], m[1], base)
            lengths = oracle.compact_range(cache, table, m[0], lengths)
            pyr.merged(lengths)
        pos = pos + np.array([x[0].shape[0] for x in per])
    assert pyr.levels == [2]
    ks = [np.concatenate([per[b][0] for per in data]) for b in range(B)]
    vs = [np.concatenate([per[b][1] for per in data]) for b in range(B)]
    ms = [np.concatenate([per[b][2] for per in data]) for b in range(B)]
    ss = [np.concatenate([[0], np.cumsum([per[b][0].shape[0] for per in data])]) for b in range(B)]
    ref = oracle.Cache("f64", B * mp, H, d)
    rcall = W._concat_call("f64", H, d, base, ks, vs, ms, ss, np.full(B, 100), table, np.zeros(B, np.int32))
    rlen = oracle.coarsen(rcall, ref, in_dtype="f64")
    np.testing.assert_array_equal(lengths, rlen)
    assert peak > int(rlen.max())                       # the pyramid gave entries back
    rk, rv, gk, gv = oracle.rows(ref.k), oracle.rows(ref.v), oracle.rows(cache.k), oracle.rows(cache.v)
    for b in range(B):
        for h in range(H):
            for e in range(-(-int(rlen[b]) // PAGE) * PAGE):
                P, s = table[b, e // PAGE], e % PAGE
                assert cache.meta[P, h, s].tobytes() == ref.meta[P, h, s].tobytes(), (b, h, e)
                np.testing.assert_allclose(gk[P, h, s], rk[P, h, s], rtol=1e-11, atol=1e-11)
                np.testing.assert_allclose(gv[P, h, s], rv[P, h, s], rtol=1e-11, atol=1e-11)
                np.testing.assert_allclose(cache.ab[P, h, s, 0], ref.ab[P, h, s, 0], rtol=1e-12)
                np.testing.assert_allclose(cache.ab[P, h, s, 1], ref.ab[P, h, s, 1], rtol=1e-10, atol=1e-13)
