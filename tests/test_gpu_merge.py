"""GPU parity of spicy_merge_level (one level of the dyadic merge) against
the CPU oracle, through the C ABI.

Both sides start every level from the same bytes (the oracle's cache so far
uploaded, metadata included).  Bars: entry kinds, masses, position sums and
alpha = bf16(ln m) bit-exact; beta within 1 unit in the last place; keys and
values within 1 unit in the last place, or within 1e-10 of the largest
magnitude in their row: both sides work in double precision and round once,
but a component that cancels to nearly zero (a rotated or averaged pair)
keeps only rounding noise of the row's scale, where the storage ulp is far
finer.  That noise is set by the rotation angles: position times frequency
reaches about 1e5 rad here, whose double-precision rounding is about 1e-11
(the GPU rotates once by tbar - tbar_i, the oracle back by tbar_i and forward
by tbar).  Nulls exact.  Then the decode of the merged GPU cache against the
decode of the merged oracle cache at the decode bars.
"""
import numpy as np
import pytest
import torch

import oracle
from coarse_grained_decode_amd import workloads as W
from test_gpu_parity import DEV, _need_gpu, compare_decode, touched_pages

pytestmark = pytest.mark.gpu

WORKLOADS = {
    "tiny_fp32": lambda: W.tiny_fp32(),
    "qwen2_1.5b_layer": lambda: W.qwen2_1p5b(),
    "qwen2_7b_small": lambda: W.qwen2_7b(B=3, T=6000),
    "long_ragged_small": lambda: W.long_ragged(T_range=(9000, 20000), B=3),
    "shared_prefix_small": lambda: W.shared_prefix(B=5, prefix_T=6000, chunk_T=2000, suffix_range=(37, 300)),
    "bf16_d64": lambda: W.qwen2_1p5b(d=64, B=4, T=4096),
    # ranges longer than one listing window of 1024 entries: about 1150
    # entries per sequence (two windows) and about 2060 (three windows)
    "qwen2_7b_two_windows": lambda: W.qwen2_7b(B=2),
    "long_ragged_three_windows": lambda: W.long_ragged(T_range=(100000, 110000), B=1),
}


def upload_with_meta(ref: oracle.Cache):
    import coarse_grained_decode_amd as cgd

    def t(a):
        if ref.store == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    meta = torch.from_numpy(np.ascontiguousarray(ref.meta).view(np.int32).reshape(ref.meta.shape + (4,))).to(DEV)
    return cgd.PagedCache(t(ref.k), t(ref.v), t(ref.ab), meta)


def gpu_merge(cache, wl, begin, end, levels=1):
    import coarse_grained_decode_amd as cgd
    tb = torch.from_numpy(np.ascontiguousarray(wl.page_table, dtype=np.int32)).to(DEV)
    eb = torch.from_numpy(np.ascontiguousarray(begin, dtype=np.int32)).to(DEV)
    ee = torch.from_numpy(np.ascontiguousarray(end, dtype=np.int32)).to(DEV)
    rng = int((np.asarray(end) - np.asarray(begin)).max()) if len(begin) else 0
    ws = cgd.workspace(cgd.spicy_merge_workspace_bytes(wl.B, wl.H_kv, rng), DEV)
    for _ in range(levels):
        cgd.spicy_merge_level(cache, wl.calls[-1].rope_base, tb, eb, ee, rng, ws)
    torch.cuda.synchronize()
    assert cgd.device_error(ws) == 0
    # after the 256-byte header, one arrival counter per (sequence, KV head):
    # every completed call leaves them at zero
    assert int(ws[64:64 + wl.B * wl.H_kv].abs().sum().item()) == 0


def store_value(bits, store):
    if store == "bf16":
        return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(bits, dtype=np.float64)


def compare_merged(gcache, ref, wl, lengths):
    from test_gpu_parity import host, ulp_dist
    store = wl.dtype
    pages = touched_pages(wl.page_table, lengths)
    gm, rm = host(gcache.meta)[pages], ref.meta[pages]
    assert np.array_equal(gm[..., 0], rm["kind"]), "entry kinds differ"
    assert np.array_equal(gm[..., 1], rm["mass"]), "masses differ"
    pos = gm[..., 2].astype(np.int64) & 0xFFFFFFFF | (gm[..., 3].astype(np.int64) << 32)
    assert np.array_equal(pos, rm["pos_sum"]), "position sums differ"
    gab, rab = host(gcache.ab)[pages], ref.ab[pages]
    assert np.array_equal(gab[..., 0], rab[..., 0]), "alpha differs"
    assert ulp_dist(gab[..., 1], rab[..., 1], store).max() <= 1, "beta differs by > 1 ulp"
    exact = {}
    for f in ("k", "v"):
        g, r = oracle.rows(host(getattr(gcache, f))[pages]), oracle.rows(getattr(ref, f)[pages])
        du = ulp_dist(g, r, store)
        gv, rv = store_value(g, store), store_value(r, store)
        scale = np.abs(rv).max(-1, keepdims=True)
        ok = (du <= 1) | (np.abs(gv - rv) <= 1e-10 * scale)
        assert ok.all(), f"{f} differs: {du.max()} ulp, worst abs {np.abs(gv - rv).max()}"
        exact[f] = float((du == 0).mean())
    return exact


def report_worst_key(gcache, ref, wl, lengths):
    """Print where the GPU and oracle keys differ most (ulps), to name a failing element."""
    from test_gpu_parity import host, ulp_dist
    pages = touched_pages(wl.page_table, lengths)
    gk, rk = oracle.rows(host(gcache.k)[pages]), oracle.rows(ref.k[pages])
    du = ulp_dist(gk, rk, wl.dtype)
    i = np.unravel_index(int(np.argmax(du)), du.shape)
    if du[i] > 1:
        mt = ref.meta[pages][i[:3]]
        print(f"[worst key] page {pages[i[0]]} head {i[1]} slot {i[2]} dim {i[3]}: {du[i]} ulp, "
              f"gpu {gk[i]} oracle {rk[i]}, kind {mt['kind']} mass {mt['mass']} pos_sum {mt['pos_sum']}; "
              f"row gpu {gk[i[:3]][:8]} oracle {rk[i[:3]][:8]}", flush=True)


def gpu_decode_plain(cache, wl, lengths):
    from test_gpu_parity import gpu_decode
    return gpu_decode(cache, wl, lengths)


@pytest.mark.parametrize("levels", [1, 2])
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_merge_matches_oracle(name, levels):
    _need_gpu()
    wl = WORKLOADS[name]()
    print(f"[merge] {name} x{levels}: B={wl.B} H_kv={wl.H_kv} d={wl.d} pages={wl.num_pages}", flush=True)
    ref = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    lengths = None
    for c in wl.calls:
        lengths = oracle.coarsen(c, ref)
    # the whole sequence, or only the per-step chunk's entries when there is one
    begin = wl.step.entry_start if wl.step is not None else np.zeros(wl.B, np.int32)
    # every level starts both sides from the same bytes (the oracle's cache
    # so far), so each comparison sees one level's arithmetic only
    for lv in range(levels):
        gcache = upload_with_meta(ref)
        oracle.merge_level(ref, wl.page_table, begin, lengths, wl.calls[-1].rope_base)
        gpu_merge(gcache, wl, begin, lengths)
        report_worst_key(gcache, ref, wl, lengths)
        ex = compare_merged(gcache, ref, wl, lengths)
        print(f"[{name}] level {lv + 1}: exact keys {ex['k']:.6f} exact values {ex['v']:.6f}")
        assert ex["k"] > 0.99 and ex["v"] > 0.99
    ro, rlse = oracle.decode(wl.q, wl.dtype, ref, wl.H_q, wl.page_table, lengths)
    o, lse = gpu_decode_plain(gcache, wl, lengths)
    compare_decode(o, lse, ro, rlse, wl.dtype)


def test_merge_of_gpu_coarsening_runs_in_the_pipeline():
    """spicy_coarsen, then spicy_merge_level over the chunk it wrote, then the
    shared-prefix decode: the same as the oracle's three steps."""
    _need_gpu()
    from coarse_grained_decode_amd.runner import DeviceWorkload
    wl = WORKLOADS["shared_prefix_small"]()
    dw = DeviceWorkload.of(wl, DEV, meta=True)
    dw.run_setup()
    dw.step.run(dw.cache)
    torch.cuda.synchronize()
    lengths = dw.step.lengths.cpu().numpy()
    gpu_merge(dw.cache, wl, wl.step.entry_start, lengths)
    dw.lengths = dw.step.lengths
    dw.decode()
    torch.cuda.synchronize()
    ref = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    for c in wl.calls:
        rlen = oracle.coarsen(c, ref)
    assert np.array_equal(rlen, lengths)
    oracle.merge_level(ref, wl.page_table, wl.step.entry_start, rlen, wl.step.rope_base)
    ro, rlse = oracle.decode(wl.q, wl.dtype, ref, wl.H_q, wl.page_table, rlen)
    compare_decode(dw.o, dw.lse, ro, rlse, wl.dtype)


def test_merge_edge_ranges():
    """Empty ranges, a range holding one macro-node, a range that starts on a
    C-point, and fp32 storage at d = 128: the same as the oracle; an empty
    call (every range empty) leaves the cache bit-identical."""
    _need_gpu()
    wl = W.qwen2_7b(B=4, T=3000, dtype="f32")
    ref = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    lengths = None
    for c in wl.calls:
        lengths = oracle.coarsen(c, ref)
    g0 = upload_with_meta(ref)
    before = {f: getattr(g0, f).clone() for f in ("k", "v", "ab", "meta")}
    gpu_merge(g0, wl, lengths, lengths)                          # every range empty
    for f, t in before.items():
        assert torch.equal(getattr(g0, f), t), f"an empty merge changed {f}"
    kinds = ref.meta["kind"]
    # sequence 0: from its second entry; 1: nothing; 2: only its first macro-node; 3: everything
    first_mac = [next(e for e in range(int(lengths[b])) if kinds[wl.page_table[b, e // 16], 0, e % 16] == 2)
                 for b in range(wl.B)]
    begin = np.array([1, 5, first_mac[2], 0], dtype=np.int32)
    end = np.array([lengths[0], 5, first_mac[2] + 1, lengths[3]], dtype=np.int32)
    gcache = upload_with_meta(ref)
    oracle.merge_level(ref, wl.page_table, begin, end, wl.calls[-1].rope_base)
    gpu_merge(gcache, wl, begin, end)
    ex = compare_merged(gcache, ref, wl, lengths)
    assert ex["k"] > 0.99 and ex["v"] > 0.99


def test_merge_rejects_diagonal_caches_and_missing_metadata():
    _need_gpu()
    import coarse_grained_decode_amd as cgd
    wl = W.qwen2_1p5b(d=64, B=4, T=4096)
    tb = torch.from_numpy(wl.page_table.astype(np.int32)).to(DEV)
    z = torch.zeros(wl.B, dtype=torch.int32, device=DEV)
    ws = cgd.workspace(cgd.spicy_merge_workspace_bytes(wl.B, wl.H_kv, 16), DEV)
    for kw, code in ((dict(meta=True, diag=True), 4), (dict(meta=False), 1)):
        cache = cgd.PagedCache.empty(wl.num_pages, wl.H_kv, wl.d, torch.bfloat16, DEV, **kw)
        with pytest.raises(cgd.SpicyError) as e:
            cgd.spicy_merge_level(cache, 1e6, tb, z, z, 16, ws)
        assert e.value.status == code


def test_merge_range_above_max_range_sets_error_and_merges_nothing():
    """A range longer than max_range raises SPICY_DEVERR_SEGMENTS and that
    (sequence, head) is left alone; max_range = 0 with every range empty is
    a no-op without error."""
    _need_gpu()
    import coarse_grained_decode_amd as cgd
    wl = W.qwen2_1p5b(d=64, B=4, T=4096)
    ref = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d)
    for c in wl.calls:
        lengths = oracle.coarsen(c, ref)
    g = upload_with_meta(ref)
    before = {f: getattr(g, f).clone() for f in ("k", "v", "ab", "meta")}
    tb = torch.from_numpy(wl.page_table.astype(np.int32)).to(DEV)
    zero = torch.zeros(wl.B, dtype=torch.int32, device=DEV)
    ln = torch.from_numpy(lengths.astype(np.int32)).to(DEV)
    for rng, end, err in ((8, ln, 0x4), (0, zero, 0)):
        ws = cgd.workspace(cgd.spicy_merge_workspace_bytes(wl.B, wl.H_kv, rng), DEV)
        cgd.spicy_merge_level(g, wl.calls[-1].rope_base, tb, zero, end, rng, ws)
        torch.cuda.synchronize()
        assert cgd.device_error(ws) == err
        for f, t in before.items():
            assert torch.equal(getattr(g, f), t), f"{f} changed"
