"""Pins of the oracle's dyadic merge level (law of total variance) against
things other than itself.

SPICY-KV demo page: the cascaded dyadic ring-buffer pyramid (Claim 12) and
the recursive law of total variance across cascades (Claim 10).  A merge
level turns each consecutive pair of macro-nodes of a (sequence, KV head)
into one macro-node of the union of their members, in place (the second entry
becomes a null).  With exact storage (f64) that must be the coarsening of the
union, which the coarsening computes directly from the tokens (two-pass
variance) and which its own pins tie to numpy.  Pins:
  * one level over fine segments = coarsening over the pairwise-joined
    segments: every non-null entry in order (keys, values, alpha, beta, mass,
    position sum), and the decode, with and without RoPE;
  * two levels = coarsening over segments joined four at a time (the
    recursive law);
  * an odd macro-node is left bit-identical; entries outside the range are
    untouched; mass is conserved and each pair leaves one null;
  * the merged variance equals numpy.var over the union's member keys;
  * a cache with the diagonal sidecar is rejected.
"""
import numpy as np
import pytest

import oracle
from coarse_grained_decode_amd import workloads as W


def build(seed, n_seg, seg_len=(6, 20), H=2, d=32, base=1e4, protect=0.1, pos_base=500):
    rng = np.random.default_rng(seed)
    lens = rng.integers(seg_len[0], seg_len[1] + 1, size=n_seg)
    T = int(lens.sum())
    segs = np.concatenate([[0], np.cumsum(lens)])
    k = rng.standard_normal((T, H, d)) + rng.standard_normal((1, H, d))
    v = rng.standard_normal((T, H, d))
    mask = rng.random((T, H)) < protect
    for s in range(n_seg):                       # every segment keeps F-tokens in every head
        mask[segs[s], :] = False
    return k, v, mask, segs, T


def call_of(k, v, mask, segs, base, pos_base=500):
    T, H, d = k.shape
    mp = -(-(2 * T + 16) // 16) + 1
    return W._concat_call("f64", H, d, base, [k], [v], [mask.astype(np.uint8)], [np.asarray(segs, np.int64)],
                          [pos_base], np.arange(mp)[None, :], [0])


def coarsen(call, meta=True):
    cache = oracle.Cache("f64", int(call.page_table.max()) + 1, call.H_kv, call.d)
    lengths = oracle.coarsen(call, cache, in_dtype="f64")
    return cache, lengths


def entries(cache, h, n):
    """Non-null entries of sequence 0, head h, in entry order (page table = identity)."""
    rk, rv = oracle.rows(cache.k), oracle.rows(cache.v)
    out = []
    for e in range(n):
        p, s = e // 16, e % 16
        mt = cache.meta[p, h, s]
        if mt["kind"] == 0:
            continue
        out.append((int(mt["kind"]), int(mt["mass"]), int(mt["pos_sum"]), rk[p, h, s], rv[p, h, s],
                    cache.ab[p, h, s, 0], cache.ab[p, h, s, 1]))
    return out


def assert_same_entries(a, b, tol=1e-12):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert x[:3] == y[:3]
        np.testing.assert_allclose(x[3], y[3], rtol=tol, atol=tol)
        np.testing.assert_allclose(x[4], y[4], rtol=tol, atol=tol)
        np.testing.assert_allclose(x[5], y[5], rtol=tol, atol=tol)
        np.testing.assert_allclose(x[6], y[6], rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("base", [1e4, 0.0])
def test_one_level_is_the_coarsening_of_joined_segments(base):
    k, v, mask, segs, T = build(1, 10)
    fine, lf = coarsen(call_of(k, v, mask, segs, base))
    coarse, lc = coarsen(call_of(k, v, mask, segs[::2], base))
    oracle.merge_level(fine, np.arange(fine.num_pages)[None, :], [0], lf, base)
    for h in range(k.shape[1]):
        assert_same_entries(entries(fine, h, int(lf[0])), entries(coarse, h, int(lc[0])))
    q = np.random.default_rng(9).standard_normal((1, 4, k.shape[2]))
    of, lsf = oracle.decode(q, "f64", fine, 4, np.arange(fine.num_pages)[None, :], lf)
    oc, lsc = oracle.decode(q, "f64", coarse, 4, np.arange(coarse.num_pages)[None, :], lc)
    np.testing.assert_allclose(of, oc, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lsf, lsc, rtol=1e-12)


def test_two_levels_are_the_coarsening_of_segments_joined_by_four():
    k, v, mask, segs, T = build(2, 12)
    base = 1e6
    fine, lf = coarsen(call_of(k, v, mask, segs, base))
    coarse, lc = coarsen(call_of(k, v, mask, segs[::4], base))
    table = np.arange(fine.num_pages)[None, :]
    oracle.merge_level(fine, table, [0], lf, base)
    oracle.merge_level(fine, table, [0], lf, base)
    for h in range(k.shape[1]):
        assert_same_entries(entries(fine, h, int(lf[0])), entries(coarse, h, int(lc[0])), tol=1e-11)


def test_odd_node_range_and_conservation():
    k, v, mask, segs, T = build(3, 7)
    base = 1e4
    c, lens = coarsen(call_of(k, v, mask, segs, base))
    before = {f: getattr(c, f).copy() for f in ("k", "v", "ab")}
    meta0 = c.meta.copy()
    # merge only the entries after the first macro-node of head 0's second segment
    n = int(lens[0])
    kinds0 = [c.meta[e // 16, 0, e % 16]["kind"] for e in range(n)]
    start = [e for e in range(n) if kinds0[e] == 2][1]
    oracle.merge_level(c, np.arange(c.num_pages)[None, :], [start], lens, base)
    for h in range(k.shape[1]):
        ms = [e for e in range(n) if meta0[e // 16, h, e % 16]["kind"] == 2 and e >= start]
        mass0 = sum(int(meta0[e // 16, h, e % 16]["mass"]) for e in range(n))
        mass1 = sum(int(c.meta[e // 16, h, e % 16]["mass"]) for e in range(n))
        assert mass0 == mass1
        nulls0 = sum(1 for e in range(n) if meta0[e // 16, h, e % 16]["kind"] == 0)
        nulls1 = sum(1 for e in range(n) if c.meta[e // 16, h, e % 16]["kind"] == 0)
        assert nulls1 - nulls0 == len(ms) // 2
        untouched = [e for e in range(n) if e < start] + ([ms[-1]] if len(ms) % 2 else [])
        for e in untouched:
            p, s = e // 16, e % 16
            assert c.meta[p, h, s] == meta0[p, h, s]
            assert np.array_equal(oracle.rows(c.k)[p, h, s], oracle.rows(before["k"])[p, h, s])
            assert np.array_equal(c.ab[p, h, s], before["ab"][p, h, s])


def test_merged_variance_is_numpy_var_of_the_union():
    rng = np.random.default_rng(4)
    d = 16
    k = rng.standard_normal((30, 1, d)) * np.linspace(0.5, 2.0, d)
    v = rng.standard_normal((30, 1, d))
    segs = [0, 11, 30]
    c, lens = coarsen(call_of(k, v, np.zeros((30, 1), bool), segs, 1e4))
    oracle.merge_level(c, np.arange(c.num_pages)[None, :], [0], lens, 1e4)
    beta = c.ab[0, 0, 0, 1]
    np.testing.assert_allclose(2 * d * beta, np.var(k[:, 0], axis=0).mean(), rtol=1e-12)
    np.testing.assert_allclose(oracle.rows(c.v)[0, 0, 0], v[:, 0].mean(0), rtol=1e-12, atol=1e-14)
    assert c.meta[0, 0, 0]["mass"] == 30 and c.meta[0, 0, 1]["kind"] == 0
    np.testing.assert_allclose(c.ab[0, 0, 0, 0], np.log(30.0), rtol=1e-15)


def test_diagonal_sidecar_is_rejected():
    k, v, mask, segs, T = build(5, 4)
    call = call_of(k, v, mask, segs, 1e4)
    cache = oracle.Cache("f64", int(call.page_table.max()) + 1, call.H_kv, call.d, diag=True)
    lens = oracle.coarsen(call, cache, in_dtype="f64")
    with pytest.raises(ValueError):
        oracle.merge_level(cache, call.page_table, [0], lens, 1e4)
