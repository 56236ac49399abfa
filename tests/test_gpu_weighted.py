"""GPU parity of spicy_coarsen_weighted (variation-weighted representatives)
against the CPU oracle, through the C ABI.

Equal-Variation KV Cache page, implementation notes: each macro-node's key and
value are sum w k / sum w and sum w v / sum w over its F-tokens (the plain
means when every weight is zero).  Bars: the coarsening bars of
test_gpu_parity (layout, mass, positions, alpha bit-exact; keys, values, beta
within 1 ulp; C-points bit copies), plus three exact invariants: equal weights
give spicy_coarsen bit for bit; weights change nothing but the macro-nodes'
keys and values (alpha, beta, metadata, lengths and the diagonal variances are
bit-identical to the unweighted call); the policy's own variation feeds it
end to end.
"""
import types

import numpy as np
import pytest
import torch

import oracle
from coarse_grained_decode_amd import workloads as W
from test_gpu_parity import DEV, _need_gpu, compare_cache, host, touched_pages

pytestmark = pytest.mark.gpu

WORKLOADS = {
    "tiny_fp32": lambda: W.tiny_fp32(),
    "qwen2_1.5b_layer": lambda: W.qwen2_1p5b(),
    "qwen2_7b_small": lambda: W.qwen2_7b(B=3, T=6000),
    "long_ragged_small": lambda: W.long_ragged(T_range=(9000, 20000), B=3),
    "bf16_d64": lambda: W.qwen2_1p5b(d=64, B=4, T=4096),
}


def gpu_run(wl, weights, diag=False):
    """Every coarsen call of the workload (setup, then step) into one fresh
    cache; weights: one array per call, or None for spicy_coarsen."""
    import dataclasses
    from coarse_grained_decode_amd.runner import DeviceCall
    import coarse_grained_decode_amd as cgd
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    cache = cgd.PagedCache.empty(wl.num_pages, wl.H_kv, wl.d, tdt, DEV, meta=True, fill=float("nan"), diag=diag)
    lengths = None
    for i, call in enumerate(wl.calls):
        dc = DeviceCall.of(call, DEV)
        if weights is not None:
            dc = dataclasses.replace(dc, token_weight=torch.from_numpy(weights[i]).to(DEV))
        dc.run(cache)
        torch.cuda.synchronize()
        assert int(dc.ws[0].item()) == 0, "device error word set"
        lengths = dc.lengths
    return cache, lengths.cpu().numpy()


def oracle_run(wl, weights, diag=False):
    cache = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d, diag=diag)
    lengths = None
    for i, call in enumerate(wl.calls):
        lengths = oracle.coarsen(call, cache, token_weight=None if weights is None else weights[i])
    return cache, lengths


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_weighted_coarsen_matches_oracle(name):
    _need_gpu()
    wl = WORKLOADS[name]()
    print(f"[weighted] {name}: B={wl.B} H_kv={wl.H_kv} d={wl.d} calls={len(wl.calls)}", flush=True)
    weights = [W.token_weights(c, 11 + i) for i, c in enumerate(wl.calls)]
    rcache, rlen = oracle_run(wl, weights)
    gcache, glen = gpu_run(wl, weights)
    assert np.array_equal(glen, rlen)
    stats = compare_cache(types.SimpleNamespace(wl=wl, cache=gcache), rcache, rlen)
    print(f"[{name}] exact keys {stats['k_exact']:.6f} exact values {stats['v_exact']:.6f}")
    assert stats["k_exact"] > 0.999 and stats["v_exact"] > 0.999


def test_equal_weights_are_spicy_coarsen_and_weights_touch_only_representatives():
    _need_gpu()
    wl = W.qwen2_7b(B=3, T=6000)
    pages = None
    plain, plen = gpu_run(wl, None, diag=True)
    ones, olen = gpu_run(wl, [np.full(c.total_tokens, 3, np.int64) for c in wl.calls], diag=True)
    rnd, rlen = gpu_run(wl, [W.token_weights(c, 21 + i) for i, c in enumerate(wl.calls)], diag=True)
    assert np.array_equal(plen, olen) and np.array_equal(plen, rlen)
    pages = touched_pages(wl.page_table, plen)
    for f in ("k", "v", "ab", "meta", "s2"):
        a, b = host(getattr(plain, f))[pages], host(getattr(ones, f))[pages]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"equal weights changed {f}"
    for f in ("ab", "meta", "s2"):
        a, b = host(getattr(plain, f))[pages], host(getattr(rnd, f))[pages]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"weights changed {f}"
    kind = host(plain.meta)[pages][..., 0]
    kp, kr = oracle.rows(host(plain.k)[pages]), oracle.rows(host(rnd.k)[pages])
    assert np.array_equal(kp[kind == 1], kr[kind == 1]), "weights changed a C-point"
    assert not np.array_equal(kp[kind == 2], kr[kind == 2])


def test_policy_variation_feeds_weighted_coarsen():
    """spicy_policy, then spicy_coarsen_weighted with the d_t the policy left
    in its workspace, against oracle_policy then oracle_coarsen_weighted."""
    _need_gpu()
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd.runner import DeviceCall, DevicePolicy
    wl = W.shared_prefix(B=5, prefix_T=6000, chunk_T=2000, suffix_range=(37, 300))
    st, pol = wl.step, wl.policy
    print(f"[weighted] policy chain: chunk {st.total_tokens} tokens", flush=True)
    ref = oracle.policy(st.k, st.v, st.seq_offsets, pol.proj_ptr, pol.proj_idx, pol.n_segments, pol.n_landmarks,
                        pol.sink, pol.recent)
    import dataclasses
    rcall = dataclasses.replace(st, seg_offsets=ref.seg_offsets, seq_seg_ptr=ref.seq_seg_ptr, mask=ref.mask)
    rcache = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    for c in wl.setup:
        oracle.coarsen(c, rcache)
    rlen = oracle.coarsen(rcall, rcache, token_weight=ref.variation)

    tdt = torch.bfloat16
    cache = cgd.PagedCache.empty(wl.num_pages, wl.H_kv, wl.d, tdt, DEV, meta=True, fill=float("nan"))
    for c in wl.setup:
        DeviceCall.of(c, DEV).run(cache)
    step = DeviceCall.of(st, DEV)
    dp = DevicePolicy.of(pol, st, DEV)
    dp.run(step)
    fed = dp.feed(step, DEV, weighted=True)
    fed.run(cache)
    torch.cuda.synchronize()
    assert int(dp.ws[0].item()) == 0 and int(fed.ws[0].item()) == 0
    assert np.array_equal(dp.variation.cpu().numpy(), ref.variation)
    glen = fed.lengths.cpu().numpy()
    assert np.array_equal(glen, rlen)
    stats = compare_cache(types.SimpleNamespace(wl=wl, cache=cache), rcache, rlen)
    assert stats["k_exact"] > 0.999 and stats["v_exact"] > 0.999


def test_weighted_with_diagonal_closure_matches_oracle():
    """Both variants at once (the streaming role's DIAG + WEIGHTED
    instantiation): the cache and the variance sidecar against the oracle."""
    _need_gpu()
    from test_gpu_diag import compare_s2
    for name in ("qwen2_7b_small", "bf16_d64"):
        wl = WORKLOADS[name]()
        print(f"[weighted+diag] {name}", flush=True)
        weights = [W.token_weights(c, 31 + i) for i, c in enumerate(wl.calls)]
        rcache, rlen = oracle_run(wl, weights, diag=True)
        gcache, glen = gpu_run(wl, weights, diag=True)
        assert np.array_equal(glen, rlen)
        stats = compare_cache(types.SimpleNamespace(wl=wl, cache=gcache), rcache, rlen)
        assert stats["k_exact"] > 0.999 and stats["v_exact"] > 0.999
        pages = touched_pages(wl.page_table, rlen)
        compare_s2(host(gcache.s2)[pages], rcache.s2[pages], rcache.meta["kind"][pages], wl.dtype)
