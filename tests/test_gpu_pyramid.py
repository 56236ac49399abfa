"""The dyadic pyramid on the GPU: chunks appended one after another with
spicy_coarsen (each at the current length) and merged by the host schedule
(runner.DyadicPyramid) with spicy_merge_level, against the oracle doing the
same steps.  The two sides evolve independently over several levels, so the
bars are: entry kinds, masses, position sums and alpha bit-exact (integer
bookkeeping and bf16(ln m)); keys and values within 1% of their row's
largest magnitude (each level rounds once to bf16 on both sides; the
per-level 1-ulp parity is tested in test_gpu_merge.py); the decode at the
decode bars.
"""
import numpy as np
import pytest
import torch

import oracle
from coarse_grained_decode_amd import workloads as W
from test_gpu_parity import DEV, _need_gpu, compare_decode, host, touched_pages
from test_pyramid import chunks

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_chunks,d", [(6, 128), (5, 64)])
def test_pyramid_matches_oracle(n_chunks, d):
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd.runner import DeviceCall, DyadicPyramid, _tensor
    _need_gpu()
    B, H, H_q, base, max_pages = 3, 2, 8, 1e6, 64
    print(f"[pyramid] {n_chunks} chunks, B={B} H={H} d={d}", flush=True)
    data = chunks(11 + d, n_chunks, B, H, d, 6, (20, 60))
    table = np.arange(B * max_pages, dtype=np.int32).reshape(B, max_pages)
    tb = _tensor(table, None, DEV)
    ref = oracle.Cache("bf16", B * max_pages, H, d)
    cache = cgd.PagedCache.empty(B * max_pages, H, d, torch.bfloat16, DEV, meta=True, fill=float("nan"))
    lengths = np.zeros(B, np.int32)
    pos = np.full(B, 100, np.int64)
    pyr = DyadicPyramid(B)
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
        merges = pyr.append(start, lengths)
        for begin, end in merges:
            oracle.merge_level(ref, table, begin, end, base)
        DyadicPyramid.run(cache, merges, base, tb, DEV)
        torch.cuda.synchronize()
        pos = pos + np.array([x[0].shape[0] for x in per])
    print(f"[pyramid] levels {pyr.levels}", flush=True)
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
