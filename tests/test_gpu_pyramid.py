"""The dyadic pyramid on the GPU: chunks appended one after another with
spicy_coarsen (each at the current length), merged by the host schedule
(runner.DyadicPyramid) with spicy_merge_level and, in the compacting modes,
given their freed entries back by spicy_compact_range after every merge.

Modes:
  plain    merges only (the cache keeps its nulls);
  compact  a compaction after every merge, called step by step;
  cascade  the same through DyadicPyramid.cascade (the runner's own loop).
In plain and compact every level is checked on its own: before each GPU
merge the GPU's bytes are read back and the oracle merges (and compacts)
that same copy, so each comparison sees one level's arithmetic only: entry
kinds, masses, position sums and alpha bit-exact; beta, keys and values
within 1 unit in the last place or within 1e-10 of their row's largest
magnitude (the merge's bar, test_gpu_merge.py); the compaction bit-exact on
every pool byte and length.  Beside it, an oracle track that coarsens,
merges and compacts from the tokens on its own gives, at the end, the same
lengths and entry bookkeeping, keys and values within 1% of their row's
largest magnitude (the levels round to bf16 independently on the two
tracks), and the decode at the decode bars.
"""
import types

import numpy as np
import pytest
import torch

import oracle
from coarse_grained_decode_amd import workloads as W
from test_gpu_compact import assert_same_pools
from test_gpu_merge import compare_merged
from test_gpu_parity import DEV, _need_gpu, compare_decode, host, touched_pages
from test_pyramid import chunks

pytestmark = pytest.mark.gpu


def download(g, store, H, d):
    """The GPU cache's bytes as an oracle cache."""
    c = oracle.Cache(store, g.num_pages, H, d, fill=False)
    c.k[:], c.v[:], c.ab[:] = host(g.k), host(g.v), host(g.ab)
    c.meta[:] = np.ascontiguousarray(host(g.meta)).reshape(-1).view(oracle.META_DTYPE).reshape(c.meta.shape)
    return c


@pytest.mark.parametrize("mode", ["plain", "compact", "cascade"])
@pytest.mark.parametrize("n_chunks,d", [(6, 128), (5, 64)])
def test_pyramid_matches_oracle(n_chunks, d, mode):
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd.runner import DeviceCall, DyadicPyramid, _tensor
    _need_gpu()
    B, H, H_q, base, max_pages = 3, 2, 8, 1e6, 64
    print(f"[pyramid] {mode}: {n_chunks} chunks, B={B} H={H} d={d}", flush=True)
    data = chunks(11 + d, n_chunks, B, H, d, 6, (20, 60))
    table = np.arange(B * max_pages, dtype=np.int32).reshape(B, max_pages)
    tb = _tensor(table, None, DEV)
    wl = types.SimpleNamespace(dtype="bf16", page_table=table)
    ref = oracle.Cache("bf16", B * max_pages, H, d)
    cache = cgd.PagedCache.empty(B * max_pages, H, d, torch.bfloat16, DEV, meta=True, fill=float("nan"))
    lengths = np.zeros(B, np.int32)
    pos = np.full(B, 100, np.int64)
    pyr = DyadicPyramid(B)
    appended = np.zeros(B, np.int64)                    # entries written, nothing given back
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    for per in data:
        bits = lambda x: W.f32_to_bf16_bits(x.astype(np.float32))
        call = W._concat_call("bf16", H, d, base, [bits(x[0]) for x in per], [bits(x[1]) for x in per],
                              [x[2] for x in per], [x[3] for x in per], pos, table, lengths)
        start = lengths.copy()
        lengths = oracle.coarsen(call, ref)
        dc = DeviceCall.of(call, DEV)
        dc.run(cache)
        torch.cuda.synchronize()
        assert int(dc.ws[0].item()) == 0
        assert np.array_equal(dc.lengths.cpu().numpy(), lengths)
        appended += lengths - start
        pyr.push(start, lengths)
        if mode == "cascade":
            # the oracle track first (it needs the schedule before the GPU runs it)
            shadow = DyadicPyramid(B)
            shadow.blocks = list(pyr.blocks)
            rlen = lengths
            while (m := shadow.next_merge()) is not None:
                oracle.merge_level(ref, table, m[0], rlen, base)
                rlen = oracle.compact_range(ref, table, m[0], rlen)
                shadow.merged(rlen)
            lengths = pyr.cascade(cache, lengths, base, tb, DEV)
            np.testing.assert_array_equal(lengths, rlen)
        while mode != "cascade" and (m := pyr.next_merge()) is not None:
            begin = m[0]
            mine = download(cache, "bf16", H, d)           # the GPU's bytes before this level
            oracle.merge_level(mine, table, begin, lengths, base)
            oracle.merge_level(ref, table, begin, lengths, base)
            rng = int((lengths - begin).max())
            ws = cgd.workspace(cgd.spicy_merge_workspace_bytes(B, H, rng), DEV)
            cgd.spicy_merge_level(cache, base, tb, _tensor(begin, None, DEV), _tensor(lengths, None, DEV), rng, ws)
            torch.cuda.synchronize()
            assert cgd.device_error(ws) == 0
            compare_merged(cache, mine, wl, lengths)
            if mode == "compact":
                mine = download(cache, "bf16", H, d)       # and before the compaction
                want = oracle.compact_range(mine, table, begin, lengths)
                out = torch.empty(B, dtype=torch.int32, device=DEV)
                cgd.spicy_compact_range(cache, tb, _tensor(begin, None, DEV), _tensor(lengths, None, DEV), out, err)
                torch.cuda.synchronize()
                assert int(err.item()) == 0
                np.testing.assert_array_equal(out.cpu().numpy(), want)
                assert_same_pools(cache, mine)
                lengths = oracle.compact_range(ref, table, begin, lengths)
                np.testing.assert_array_equal(lengths, want)
                pyr.merged(lengths)
            else:
                pyr.merged()
        pos = pos + np.array([x[0].shape[0] for x in per])
    print(f"[pyramid] levels {pyr.levels}, lengths {lengths.tolist()} (appended {appended.tolist()})", flush=True)
    if mode == "plain":
        np.testing.assert_array_equal(lengths, appended)
    else:
        assert (lengths < appended).all()                  # the merges gave entries back
    gm, rm = host(cache.meta), ref.meta
    used = touched_pages(table, lengths)            # pages below each sequence's length
    assert np.array_equal(gm[used][..., 0], rm["kind"][used])
    assert np.array_equal(gm[used][..., 1], rm["mass"][used])
    pos_g = gm[used][..., 2].astype(np.int64) & 0xFFFFFFFF | (gm[used][..., 3].astype(np.int64) << 32)
    assert np.array_equal(pos_g, rm["pos_sum"][used])
    assert np.array_equal(host(cache.ab)[used][..., 0], ref.ab[used][..., 0])
    for f in ("k", "v"):
        g = oracle.rows(host(getattr(cache, f))[used])
        r = oracle.rows(getattr(ref, f)[used])
        gv = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rv = (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        scale = np.abs(rv).max(-1, keepdims=True)
        assert (np.abs(gv - rv) <= 1e-2 * scale).all(), f"{f} differs"
    q = np.random.default_rng(5).standard_normal((B, H_q, d)).astype(np.float32)
    qb = W.f32_to_bf16_bits(q)
    ro, rlse = oracle.decode(qb, "bf16", ref, H_q, table, lengths)
    o = torch.empty(B, H_q, d, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=DEV)
    ws = cgd.workspace(cgd.spicy_decode_workspace_bytes(B, H_q, H, d, max_pages, 0), DEV)
    cgd.spicy_decode_attn(cache, _tensor(qb, "bf16", DEV), tb, _tensor(lengths, None, DEV), o, lse, ws)
    torch.cuda.synchronize()
    assert cgd.device_error(ws) == 0
    compare_decode(o, lse, ro, rlse, "bf16")
