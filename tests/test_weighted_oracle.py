"""Pins of the oracle's variation-weighted representatives against things
other than itself.

Equal-Variation KV Cache page, implementation notes: each segment keeps a
representative key and value, the variation-weighted averages
sum_r d_r k_r / sum_r d_r (values alike).  In a SPICY-KV macro-node the
representative replaces the plain mean of the F-tokens; mass, alpha, the
anchor, beta and the diagonal variances keep their plain definitions, and a
segment whose weights are all zero keeps the plain mean.  Pins:
  * equal (or proportional) weights give the plain result bit for bit;
  * one non-zero weight gives that token's value exactly and its key rotated
    to the segment's anchor;
  * two weighted tokens, no rotation: the closed form (w1 k1 + w2 k2)/(w1 + w2);
  * all-zero weights: the plain result;
  * weights never change mass, alpha, beta, positions, lengths or s2;
  * the policy's own variation as weights, against numpy.average per segment
    on random data;
  * a negative weight is rejected.
"""
import numpy as np
import pytest

import oracle
from coarse_grained_decode_amd import workloads as W


def call_of(k, v, mask, segs, base=0.0, pos_base=0):
    T, H, d = k.shape
    return W._concat_call("f64", H, d, base, [k], [v], [np.asarray(mask, dtype=np.uint8).reshape(T, H)],
                          [np.asarray(segs, dtype=np.int64)], [pos_base],
                          np.arange(-(-(T + 16) // 16) + 1)[None, :], [0])


def run(call, weights=None, diag=False):
    cache = oracle.Cache("f64", int(call.page_table.max()) + 1, call.H_kv, call.d, diag=diag)
    lengths = oracle.coarsen(call, cache, in_dtype="f64", token_weight=weights)
    return cache, lengths


def random_case(seed, T=120, H=2, d=32, base=1e4):
    rng = np.random.default_rng(seed)
    # dyadic rationals with few bits (like bf16 data): every sum and weighted
    # sum below is exact in double precision, so equal results are bit-equal
    k = np.round(rng.standard_normal((T, H, d)) * 64) / 64
    v = np.round(rng.standard_normal((T, H, d)) * 64) / 64
    mask = rng.random((T, H)) < 0.15
    segs = [0] + sorted(rng.choice(np.arange(1, T), size=7, replace=False).tolist()) + [T]
    return call_of(k, v, mask, segs, base=base, pos_base=321), k, v, mask, segs


def same(a, b):
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_equal_and_proportional_weights_are_the_plain_mean():
    call, *_ = random_case(1)
    c0, l0 = run(call)
    for w in (np.full(call.k.shape[0], 1), np.full(call.k.shape[0], 37)):
        c1, l1 = run(call, w)
        assert np.array_equal(l0, l1)
        for f in ("k", "v", "ab"):
            assert same(getattr(c0, f), getattr(c1, f)), f
    # proportional weights: w and 4w give the same representatives
    w = np.random.default_rng(2).integers(0, 1000, size=call.k.shape[0])
    ca, _ = run(call, w)
    cb, _ = run(call, 4 * w)
    for f in ("k", "v", "ab"):
        assert same(getattr(ca, f), getattr(cb, f)), f


def test_one_weighted_token_is_that_token():
    d, base, pos_base = 16, 1e4, 900
    rng = np.random.default_rng(4)
    k = np.round(rng.standard_normal((6, 1, d)) * 64) / 64     # 5 x and 5 x / 5 exact
    v = np.round(rng.standard_normal((6, 1, d)) * 64) / 64
    w = np.array([0, 0, 5, 0, 0, 0])
    c, _ = run(call_of(k, v, np.zeros((6, 1)), [0, 6], base=base, pos_base=pos_base), w)
    kr, vr = oracle.rows(c.k)[0, 0, 0], oracle.rows(c.v)[0, 0, 0]
    assert np.array_equal(vr, v[2, 0])
    tbar = pos_base + 2.5                                    # the anchor stays the plain mean position
    np.testing.assert_allclose(kr, oracle.rope(k[2, 0], tbar, base), rtol=0, atol=1e-15)
    assert c.meta["mass"][0, 0, 0] == 6


def test_two_weighted_tokens_closed_form():
    d = 8
    k = np.array([[1.0] * d, [4.0] * d])[:, None, :] * np.arange(1, d + 1)
    v = np.array([[2.0] * d, [-1.0] * d])[:, None, :]
    c, _ = run(call_of(k, v, np.zeros((2, 1)), [0, 2], base=0.0), np.array([1, 2]))
    np.testing.assert_array_equal(oracle.rows(c.k)[0, 0, 0], (1 * k[0, 0] + 2 * k[1, 0]) / 3)
    np.testing.assert_array_equal(oracle.rows(c.v)[0, 0, 0], np.zeros(d))     # (2 - 2) / 3


def test_zero_weights_keep_the_plain_mean():
    call, *_ = random_case(5)
    c0, _ = run(call)
    c1, _ = run(call, np.zeros(call.k.shape[0], dtype=np.int64))
    for f in ("k", "v", "ab"):
        assert same(getattr(c0, f), getattr(c1, f)), f


def test_weights_change_only_the_representatives():
    call, *_ = random_case(6)
    w = np.random.default_rng(7).integers(0, 50, size=call.k.shape[0])
    c0, l0 = run(call, diag=True)
    c1, l1 = run(call, w, diag=True)
    assert np.array_equal(l0, l1)
    assert same(c0.ab, c1.ab)
    assert np.array_equal(c0.meta, c1.meta)
    assert same(c0.s2, c1.s2)
    macro = c0.meta["kind"] == 2
    assert not np.array_equal(oracle.rows(c0.k)[macro], oracle.rows(c1.k)[macro])
    cp = c0.meta["kind"] == 1                                # C-points are exact either way
    assert same(oracle.rows(c0.k)[cp], oracle.rows(c1.k)[cp])


def test_policy_variation_as_weights_against_numpy_average():
    c = W.random_policy_case(3, B=2, T_range=(60, 140), H=2, d=64, n_segments=6, n_landmarks=3, sink=1, recent=2)
    pr = oracle.policy(c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, 6, 3, 1, 2)
    T, H, d = c.k.shape
    B = len(c.seq_offsets) - 1
    lens = np.diff(c.seq_offsets)
    mp = int(-(-(lens.max() + 16) // 16)) + 1
    table = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
    call = W.CoarsenCall("bf16", H, d, 0.0, c.k, c.v, c.seq_offsets.astype(np.int32), np.zeros(B, np.int32),
                         pr.seg_offsets, pr.seq_seg_ptr, pr.mask, table, np.zeros(B, np.int32))
    cache = oracle.Cache("f64", B * mp, H, d)
    oracle.coarsen(call, cache, in_dtype="bf16", token_weight=pr.variation)
    kf = (c.k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vf = (c.v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rows_k, rows_v = oracle.rows(cache.k), oracle.rows(cache.v)
    checked = 0
    for b in range(B):
        for h in range(H):
            e = 0
            for s in range(pr.seq_seg_ptr[b], pr.seq_seg_ptr[b + 1]):
                a, z = pr.seg_offsets[s], pr.seg_offsets[s + 1]
                f = [t for t in range(a, z) if not pr.mask[t, h]]
                if f:
                    w = pr.variation[f].astype(np.float64)
                    wk = np.average(kf[f, h], axis=0, weights=w) if w.sum() > 0 else kf[f, h].mean(0)
                    wv = np.average(vf[f, h], axis=0, weights=w) if w.sum() > 0 else vf[f, h].mean(0)
                    P, slot = table[b, e // 16], e % 16
                    np.testing.assert_allclose(rows_k[P, h, slot], wk, rtol=1e-12, atol=1e-12)
                    np.testing.assert_allclose(rows_v[P, h, slot], wv, rtol=1e-12, atol=1e-12)
                    checked += 1
                    e += 1
                e += sum(1 for t in range(a, z) if pr.mask[t, h])
    assert checked > 10


def test_negative_weight_is_rejected():
    call, *_ = random_case(8)
    w = np.ones(call.k.shape[0], dtype=np.int64)
    w[3] = -1
    if call.mask[3].all():
        w[3], w[4] = 1, -1
    with pytest.raises(ValueError):
        run(call, w)
