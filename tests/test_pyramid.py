"""The host-side dyadic pyramid schedule (runner.DyadicPyramid) and, on the
oracle, what it composes to.

SPICY-KV demo page, Claims 10 and 12: a cascade of dyadic levels whose
variances combine by the law of total variance.  Pins:
  * the schedule is a binary counter: after n appended chunks the block
    levels are the binary digits of n, and n - popcount(n) merges ran;
  * with exact storage, four chunks of four segments each, appended and
    merged by the schedule, equal the coarsening of the same tokens with one
    segment per chunk (every non-null entry in order, and the decode), with
    and without RoPE: a level-2 node covers four base segments.
"""
import numpy as np
import pytest

import oracle
from coarse_grained_decode_amd import workloads as W
from coarse_grained_decode_amd.runner import DyadicPyramid


def test_schedule_is_a_binary_counter():
    p = DyadicPyramid(3)
    merges = 0
    for n in range(1, 40):
        b = np.full(3, 10 * (n - 1), np.int32)
        ms = p.append(b, b + 10)
        merges += len(ms)
        want = [i for i in range(6, -1, -1) if n >> i & 1]
        assert p.levels == want, (n, p.levels)
        assert merges == n - bin(n).count("1")
        for begin, end in ms:                         # merges cover whole, adjacent blocks
            assert (begin < end).all()
    # the last merge of a cascade spans everything merged so far
    p = DyadicPyramid(1)
    for n in range(8):
        ms = p.append(np.array([4 * n]), np.array([4 * n + 4]))
    assert ms[-1][0][0] == 0 and ms[-1][1][0] == 32


def chunks(seed, n_chunks, B, H, d, seg_per_chunk, seg_len):
    """Seeded chunks: per chunk and sequence, keys, values, a protection mask
    (10%, never a segment's first token) and segment offsets."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n_chunks):
        per = []
        for b in range(B):
            lens = rng.integers(seg_len[0], seg_len[1] + 1, size=seg_per_chunk)
            T = int(lens.sum())
            segs = np.concatenate([[0], np.cumsum(lens)])
            k = rng.standard_normal((T, H, d)) + rng.standard_normal((1, H, d))
            v = rng.standard_normal((T, H, d))
            mask = rng.random((T, H)) < 0.1
            mask[segs[:-1], :] = False
            per.append((k, v, mask, segs))
        out.append(per)
    return out


def run_pyramid(store, data, B, H, d, base, max_pages, in_dtype):
    """Coarsen the chunks one after another (each appended at the current
    length), merging by the schedule after each; returns cache, lengths."""
    table = np.arange(B * max_pages, dtype=np.int32).reshape(B, max_pages)
    cache = oracle.Cache(store, B * max_pages, H, d)
    lengths = np.zeros(B, np.int32)
    pos = np.full(B, 100, np.int64)
    pyr = DyadicPyramid(B)
    for per in data:
        call = W._concat_call(store if in_dtype is None else in_dtype, H, d, base, [x[0] for x in per],
                              [x[1] for x in per], [x[2] for x in per], [x[3] for x in per], pos, table, lengths)
        start = lengths.copy()
        lengths = oracle.coarsen(call, cache, in_dtype=in_dtype)
        for begin, end in pyr.append(start, lengths):
            oracle.merge_level(cache, table, begin, end, base)
        pos = pos + np.array([x[0].shape[0] for x in per])
    return cache, lengths, table


def nonnull(cache, table, b, h, n):
    rk, rv = oracle.rows(cache.k), oracle.rows(cache.v)
    out = []
    for e in range(n):
        p, s = table[b, e // 16], e % 16
        mt = cache.meta[p, h, s]
        if mt["kind"] != 0:
            out.append((int(mt["kind"]), int(mt["mass"]), int(mt["pos_sum"]), rk[p, h, s], rv[p, h, s],
                        cache.ab[p, h, s]))
    return out


@pytest.mark.parametrize("base", [1e4, 0.0])
def test_four_chunks_compose_to_one_segment_per_chunk(base):
    B, H, d = 2, 2, 32
    data = chunks(7, 4, B, H, d, 4, (5, 12))
    cache, lengths, table = run_pyramid("f64", data, B, H, d, base, 40, "f64")
    # the same tokens in one call, one segment per chunk
    ks, vs, ms, ss = [], [], [], []
    for b in range(B):
        ks.append(np.concatenate([per[b][0] for per in data]))
        vs.append(np.concatenate([per[b][1] for per in data]))
        ms.append(np.concatenate([per[b][2] for per in data]))
        Ts = [per[b][0].shape[0] for per in data]
        ss.append(np.concatenate([[0], np.cumsum(Ts)]))
    table2 = np.arange(B * 40, dtype=np.int32).reshape(B, 40)
    ref = oracle.Cache("f64", B * 40, H, d)
    call = W._concat_call("f64", H, d, base, ks, vs, ms, ss, np.full(B, 100), table2, np.zeros(B, np.int32))
    rlen = oracle.coarsen(call, ref, in_dtype="f64")
    for b in range(B):
        for h in range(H):
            got, want = nonnull(cache, table, b, h, int(lengths[b])), nonnull(ref, table2, b, h, int(rlen[b]))
            assert len(got) == len(want)
            for x, y in zip(got, want):
                assert x[:3] == y[:3]
                np.testing.assert_allclose(x[3], y[3], rtol=1e-11, atol=1e-11)
                np.testing.assert_allclose(x[4], y[4], rtol=1e-11, atol=1e-11)
                np.testing.assert_allclose(x[5], y[5], rtol=1e-10, atol=1e-13)
    q = np.random.default_rng(3).standard_normal((B, 4, d))
    o1, l1 = oracle.decode(q, "f64", cache, 4, table, lengths)
    o2, l2 = oracle.decode(q, "f64", ref, 4, table2, rlen)
    np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)
