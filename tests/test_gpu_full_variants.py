"""The next-row variants at the benchmark's full size (the `shared_prefix`
workload: 32 sequences, a 65536-token shared prefix, an 8192-token chunk per
sequence), in the launch configuration bench.py times, against the oracle
run on the whole workload.  Bars as in the per-variant test files: the
coarsening bars (layout bit-exact, values within 1 ulp, >= 99.9% of keys
and values bit-exact), the diagonal variances within 1 ulp or 1e-12 of their
trace, merged rows within 1 ulp or 1e-10 of their row, and the decode bars.
"""
import dataclasses
import types

import numpy as np
import pytest
import torch

import oracle
from coarse_grained_decode_amd import workloads as W
from test_gpu_parity import DEV, _need_gpu, compare_cache, compare_decode, host, touched_pages

pytestmark = pytest.mark.gpu


def _workload():
    return W.shared_prefix()


def test_full_diagonal_closure():
    _need_gpu()
    from coarse_grained_decode_amd.runner import DeviceWorkload
    from test_gpu_diag import compare_s2
    wl = _workload()
    print(f"[full diag] {wl.name}", flush=True)
    rcache, rlen, ro, rlse = oracle.run_workload(wl, diag=True)
    dw = DeviceWorkload.of(wl, DEV, diag=True)
    dw.run_setup()
    dw.step_once()
    torch.cuda.synchronize()
    assert np.array_equal(dw.lengths.cpu().numpy(), rlen)
    stats = compare_cache(dw, rcache, rlen)
    assert stats["k_exact"] > 0.999 and stats["v_exact"] > 0.999
    pages = touched_pages(wl.page_table, rlen)
    compare_s2(host(dw.cache.s2)[pages], rcache.s2[pages], rcache.meta["kind"][pages], wl.dtype)
    compare_decode(dw.o, dw.lse, ro, rlse, wl.dtype)


def test_full_policy_with_weighted_representatives():
    _need_gpu()
    from coarse_grained_decode_amd.runner import DeviceWorkload, DevicePolicy
    wl = _workload()
    st, pol = wl.step, wl.policy
    print(f"[full weighted] {wl.name}", flush=True)
    ref = oracle.policy(st.k, st.v, st.seq_offsets, pol.proj_ptr, pol.proj_idx, pol.n_segments, pol.n_landmarks,
                        pol.sink, pol.recent)
    rcall = dataclasses.replace(st, seg_offsets=ref.seg_offsets, seq_seg_ptr=ref.seq_seg_ptr, mask=ref.mask)
    rcache = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    for c in wl.setup:
        oracle.coarsen(c, rcache)
    rlen = oracle.coarsen(rcall, rcache, token_weight=ref.variation)
    ro, rlse = oracle.decode(wl.q, wl.dtype, rcache, wl.H_q, wl.page_table, rlen)

    dw = DeviceWorkload.of(wl, DEV)
    dw.run_setup()
    dp = DevicePolicy.of(pol, dw.step.call, DEV)
    dp.run(dw.step)
    fed = dp.feed(dw.step, DEV, weighted=True)
    fed.run(dw.cache)
    dw.lengths = fed.lengths
    dw.decode()
    torch.cuda.synchronize()
    assert int(dp.ws[0].item()) == 0 and int(fed.ws[0].item()) == 0
    assert np.array_equal(fed.lengths.cpu().numpy(), rlen)
    stats = compare_cache(types.SimpleNamespace(wl=wl, cache=dw.cache), rcache, rlen)
    assert stats["k_exact"] > 0.999 and stats["v_exact"] > 0.999
    compare_decode(dw.o, dw.lse, ro, rlse, wl.dtype)


def test_full_merge_level():
    _need_gpu()
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd.runner import DeviceWorkload
    from test_gpu_merge import compare_merged
    wl = _workload()
    print(f"[full merge] {wl.name}", flush=True)
    rcache = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    for c in wl.calls:
        rlen = oracle.coarsen(c, rcache)
    oracle.merge_level(rcache, wl.page_table, wl.step.entry_start, rlen, wl.step.rope_base)
    ro, rlse = oracle.decode(wl.q, wl.dtype, rcache, wl.H_q, wl.page_table, rlen)

    dw = DeviceWorkload.of(wl, DEV, meta=True)
    dw.run_setup()
    dw.step.run(dw.cache)
    st = dw.step
    rng = int(np.diff(st.call.seq_offsets).max()) + int(np.diff(st.call.seq_seg_ptr).max()) + 16
    ws = cgd.workspace(cgd.spicy_merge_workspace_bytes(wl.B, wl.H_kv, rng), DEV)
    cgd.spicy_merge_level(dw.cache, st.call.rope_base, st.page_table, st.entry_start, st.lengths, rng, ws,
                          max_pages_per_seq=st.call.max_pages)
    dw.lengths = st.lengths
    dw.decode()
    torch.cuda.synchronize()
    assert cgd.device_error(ws) == 0
    glen = st.lengths.cpu().numpy()
    assert np.array_equal(glen, rlen)
    # the coarsening step itself is bit-for-bit the tested one; the merged
    # rows carry the merge's own rounding
    ex = compare_merged(dw.cache, rcache, wl, rlen)
    assert ex["k"] > 0.99 and ex["v"] > 0.99
    compare_decode(dw.o, dw.lse, ro, rlse, wl.dtype)


def test_full_four_query_tokens():
    _need_gpu()
    from coarse_grained_decode_amd.runner import DeviceWorkload
    wl = _workload()
    print(f"[full q4] {wl.name}", flush=True)
    rcache = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    for c in wl.calls:
        rlen = oracle.coarsen(c, rcache)
    q4 = W.query_tokens(wl, 4)
    ro, rlse = oracle.decode_multi(q4, wl.dtype, rcache, wl.page_table, rlen)
    dw = DeviceWorkload.of(wl, DEV, q_tokens=4)
    dw.run_setup()
    dw.step_once()
    torch.cuda.synchronize()
    B, H_q, d = wl.B, wl.H_q, wl.d
    compare_decode(dw.o.reshape(B * 4, H_q, d), dw.lse.reshape(B * 4, H_q),
                   ro.reshape(B * 4, H_q, d), rlse.reshape(B * 4, H_q), wl.dtype)
