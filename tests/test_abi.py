"""The C ABI on the host: the library loads, exports every function declared in
include/spicy.h, and rejects bad arguments before launching anything (these
calls never reach the GPU, so they run anywhere)."""
import ctypes
import os
import re

import pytest

import coarse_grained_decode_amd as cgd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spicy.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spicy_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cgd.library_path()):
        from coarse_grained_decode_amd import build
        build.build(verbose=False)
    return cgd.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"spicy_coarsen", "spicy_decode_attn", "spicy_coarsen_workspace_bytes",
            "spicy_decode_workspace_bytes", "spicy_decode_num_splits", "spicy_status_string",
            "spicy_decode_attn_shared", "spicy_decode_shared_workspace_bytes",
            "spicy_policy", "spicy_policy_workspace_bytes",
            "spicy_decode_attn_multi", "spicy_decode_multi_workspace_bytes",
            "spicy_coarsen_weighted", "spicy_merge_level", "spicy_merge_workspace_bytes",
            "spicy_decode_plan"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(6):
        assert cgd.spicy_status_string(code).startswith("SPICY_")
    assert "unknown" in cgd.spicy_status_string(99)


def test_workspace_and_split_plan(lib):
    # split plan: explicit counts are honoured up to the page count; the
    # effective count never leaves an empty split
    assert cgd.spicy_decode_num_splits(1, 1, 10, 4) == 4
    assert cgd.spicy_decode_num_splits(1, 1, 10, 6) == 5          # 2 pages each
    assert cgd.spicy_decode_num_splits(1, 1, 3, 100) == 3
    assert cgd.spicy_decode_num_splits(4, 4, 0, 0) == 1
    for B, H, P in ((16, 4, 72), (8, 4, 164), (32, 4, 290), (8, 2, 24), (1, 1, 8)):
        s = cgd.spicy_decode_num_splits(B, H, P, 0)
        pps = -(-P // s)
        assert 1 <= s <= P and -(-P // pps) == s
        # a page group is one workgroup of 4 wavefronts: about 192 groups over
        # the call's (sequence, KV head) units, at least one page per
        # wavefront, cut so that no group is empty
        want = max(1, min(-(-192 // (B * H)), max(1, P // 4)))
        n = max(1, min(want, P))
        assert s == -(-P // -(-P // n))
        assert pps >= min(4, P) or s == 1
    up = lambda x: (x + 255) // 256 * 256

    def ws(B, n_q, H_q, d, slots):
        # header, one int32 ticket per query row, then per (row, slot) the
        # (max, sum) pair and the d-float unnormalised output
        rows = B * n_q * H_q
        return 256 + up(4 * rows) + up(8 * rows * slots) + up(4 * rows * slots * d)

    def f32_groups(maxp, ns):
        n = min(ns, 256) if ns > 0 else -(-maxp // 16)
        n = max(1, min(n, maxp))
        return -(-maxp // -(-maxp // n))

    # 8 explicit splits: 8 private groups on both kernels
    assert cgd.spicy_decode_workspace_bytes(16, 28, 4, 128, 72, 8) == ws(16, 1, 28, 128, 8)
    # shared prefix: slots = prefix groups + private groups (bf16), or the fp32
    # kernel's groups over every page, whichever is larger
    pl = cgd.spicy_decode_plan(32, 28, 4, 241, 144, 8)
    assert pl["private_splits"] == 8
    slots = max(pl["prefix_chunks"] + pl["private_splits"], f32_groups(241, 8))
    assert cgd.spicy_decode_shared_workspace_bytes(32, 28, 4, 128, 241, 144, 8) == ws(32, 1, 28, 128, slots)
    # fp32 caches ignore the prefix, so the size covers the plain plan too
    assert cgd.spicy_decode_shared_workspace_bytes(2, 4, 2, 64, 40, 39, 5) >= \
        cgd.spicy_decode_workspace_bytes(2, 4, 2, 64, 40, 5)
    assert cgd.spicy_decode_shared_workspace_bytes(2, 4, 2, 64, 40, 1, 40) >= \
        cgd.spicy_decode_workspace_bytes(2, 4, 2, 64, 40, 40)
    assert cgd.spicy_decode_shared_workspace_bytes(2, 4, 2, 64, 40, 0, 0) == \
        cgd.spicy_decode_workspace_bytes(2, 4, 2, 64, 40, 0)
    assert cgd.spicy_decode_shared_workspace_bytes(2, 4, 2, 64, 40, -1, 0) == 0
    # header, 16 B per segment, 8 B per (segment, head), 8 B per C-point
    # item (at most tokens x heads), 4 B per sequence and per (sequence,
    # head), then staged macro-nodes: key and value rows, alpha/beta, 16 B
    # of metadata, and the per-dimension variance row (diagonal closure)
    stage = 3 * up(40 * 128 * 2) + up(40 * 2 * 2) + up(40 * 16)
    assert cgd.spicy_coarsen_workspace_bytes(2, 10, 100, 4, 128, 1) == 256 + 256 + 512 + 3328 + 256 + 256 + stage
    assert cgd.spicy_coarsen_workspace_bytes(-1, 10, 100, 4, 128, 1) == 0
    assert cgd.spicy_coarsen_workspace_bytes(2, 10, -1, 4, 128, 1) == 0
    assert cgd.spicy_coarsen_workspace_bytes(2, 10, 100, 4, 128, 7) == 0


def _cache(dtype=1, H=4, d=128, pages=8, k=1, v=1, ab=1):
    return cgd._Cache(dtype, H, d, pages, k, v, ab, None)


def test_decode_rejects_bad_arguments(lib):
    P = 0x1000  # never dereferenced: validation fails before any launch
    c = _cache()

    def call(cache=c, q=P, hq=28, table=P, maxp=8, lengths=P, B=2, o=P, lse=P, ws=P, wsb=1 << 30, ns=0):
        return lib.spicy_decode_attn(ctypes.byref(cache) if cache is not None else None, q, hq, table, maxp,
                                     lengths, B, o, lse, ws, wsb, ns, None)

    assert call(cache=None) == 1
    assert call(cache=_cache(dtype=7)) == 1
    assert call(cache=_cache(d=96)) == 4
    assert call(cache=_cache(H=65)) == 4
    assert call(cache=_cache(k=0)) == 1
    assert call(hq=30) == 4                 # not a multiple of H_kv
    assert call(hq=4 * 17) == 4             # group of 17 > 16
    assert call(q=0) == 1
    assert call(lengths=0) == 1
    assert call(o=0) == 1
    assert call(ws=0) == 1
    assert call(maxp=0) == 1
    assert call(B=-1) == 1
    assert call(ns=-2) == 1
    assert call(wsb=16) == 3
    assert call(B=0, q=0, table=0) == 0     # nothing to do


def test_shared_decode_rejects_bad_arguments(lib):
    P = 0x1000
    c = _cache()

    def call(shared, maxp=8, wsb=1 << 30, cache=c):
        return lib.spicy_decode_attn_shared(ctypes.byref(cache), P, 28, P, maxp, P, 2, shared, P, P, P, wsb, 0,
                                            None)

    assert call(-1) == 1
    assert call(9) == 2                     # more shared pages than the table has
    assert call(4, wsb=16) == 3
    assert call(4, cache=_cache(d=96)) == 4


def test_coarsen_rejects_bad_arguments(lib):
    P = 0x1000
    c = _cache()

    def call(cache=c, k=P, v=P, total=100, so=P, pb=P, seg=P, ssp=P, nseg=10, mask=P, B=2, table=P, maxp=8,
             es=P, lo=P, ws=P, wsb=1 << 30):
        return lib.spicy_coarsen(ctypes.byref(cache) if cache is not None else None, k, v, total, so, pb, seg,
                                 ssp, nseg, mask, B, 1e4, table, maxp, es, lo, ws, wsb, None)

    assert call(cache=None) == 1
    assert call(cache=_cache(d=32)) == 4
    assert call(k=0) == 1
    assert call(mask=0) == 1
    assert call(so=0) == 1
    assert call(lo=0) == 1
    assert call(ws=0) == 1
    assert call(B=-3) == 1
    assert call(nseg=-1) == 1
    assert call(total=-1) == 1
    assert call(maxp=0) == 1
    assert call(maxp=(1 << 23) + 1) == 4   # entry ids would not fit a C-point item
    assert call(cache=_cache(pages=0)) == 2
    assert call(wsb=100) == 3
    assert call(B=0) == 0


def test_weighted_coarsen_rejects_bad_arguments(lib):
    P = 0x1000
    c = _cache()

    def call(w=P, total=100, B=2, k=P, wsb=1 << 30):
        return lib.spicy_coarsen_weighted(ctypes.byref(c), k, P, total, P, P, P, P, 10, P, w, B, 1e4, P, 8, P, P, P,
                                          wsb, None)

    assert call(w=0) == 1                   # weights are required when there are tokens
    assert call(k=0) == 1
    assert call(B=-1) == 1
    assert call(wsb=100) == 3
    assert call(w=0, B=0) == 0
    assert call(w=0, total=0, B=0) == 0


def test_decode_plan(lib):
    """spicy_decode_plan: the plain decode's private splits are
    spicy_decode_num_splits; a prefix gets chunks that cover it; errors."""
    for B, H_kv, maxp, ns in [(32, 4, 200, 0), (3, 2, 17, 0), (32, 4, 200, 16), (1, 1, 1, 0), (64, 8, 9000, 5)]:
        pl = cgd.spicy_decode_plan(B, 4 * H_kv, H_kv, maxp, 0, ns)
        assert pl["prefix_chunks"] == 0 and pl["prefix_chunk_pages"] == 0
        assert pl["private_splits"] == lib.spicy_decode_num_splits(B, H_kv, maxp, ns)
        assert pl["private_splits"] * pl["private_pages_per_split"] >= maxp
        assert (pl["private_splits"] - 1) * pl["private_pages_per_split"] < maxp
    pl = cgd.spicy_decode_plan(32, 28, 4, 300, 144, 0)
    assert pl["prefix_chunks"] * pl["prefix_chunk_pages"] >= 144
    assert (pl["prefix_chunks"] - 1) * pl["prefix_chunk_pages"] < 144
    assert pl["private_splits"] * pl["private_pages_per_split"] >= 300 - 144
    assert cgd.spicy_decode_plan(2, 8, 2, 10, 10, 0)["private_splits"] == 0   # prefix only
    out = (ctypes.c_int32 * 4)()
    assert lib.spicy_decode_plan(2, 8, 2, 10, 11, 0, 1, out) == 2           # prefix longer than the table
    assert lib.spicy_decode_plan(2, 8, 2, 10, 0, 0, 0, out) == 1            # no query tokens
    assert lib.spicy_decode_plan(2, 8, 2, 10, 0, 0, 1, None) == 1


def test_merge_rejects_bad_arguments(lib):
    P = 0x1000
    c = _cache()
    c.meta = P

    def call(cache=c, B=2, tb=P, eb=P, ee=P, rng=100, ws=P, wsb=1 << 30):
        return lib.spicy_merge_level(ctypes.byref(cache) if cache is not None else None, B, 1e4, tb, 8, eb, ee, rng,
                                     ws, wsb, None)

    assert call(cache=None) == 1
    assert call(B=-1) == 1
    assert call(rng=-1) == 1
    assert call(tb=0) == 1
    assert call(ee=0) == 1
    assert call(ws=0) == 1
    assert call(wsb=64) == 3
    assert call(B=20000) == 4               # B * H_kv above the 65535 units of the pair grid
    assert call(B=0) == 0
    nometa = _cache()
    assert call(cache=nometa) == 1          # the metadata (exact masses, anchors) is required
    diag = _cache()
    diag.meta, diag.s2 = P, P
    assert call(cache=diag) == 4
    # header, int32 count per (sequence, head), int4 per pair, (range + 1) / 2 pairs
    up = lambda x: (x + 255) // 256 * 256
    assert lib.spicy_merge_workspace_bytes(3, 4, 101) == 256 + up(4 * 12)
    assert lib.spicy_merge_workspace_bytes(3, 0, 101) == 0


def test_multi_decode_rejects_bad_arguments(lib):
    P = 0x1000
    c = _cache()

    def call(nq, B=2, shared=0, wsb=1 << 30):
        return lib.spicy_decode_attn_multi(ctypes.byref(c), P, nq, 28, P, 8, P, B, shared, P, P, P, wsb, 0, None)

    assert call(0) == 1
    assert call(-2) == 1
    assert call(3, B=40000) == 4            # B * tokens above the 65535 rows of the combine grid
    assert call(3, wsb=16) == 3
    assert call(3, shared=9) == 2
    # a single token needs exactly the shared decode's workspace; more tokens more
    one = lib.spicy_decode_multi_workspace_bytes(2, 1, 28, 4, 128, 8, 3, 0)
    assert one == lib.spicy_decode_shared_workspace_bytes(2, 28, 4, 128, 8, 3, 0)
    assert lib.spicy_decode_multi_workspace_bytes(2, 4, 28, 4, 128, 8, 3, 0) > one
    assert lib.spicy_decode_multi_workspace_bytes(2, 0, 28, 4, 128, 8, 3, 0) == 0


def test_policy_workspace_and_bad_arguments(lib):
    # header, then int64 d_t per token and uint64 key norms per (token, head)
    assert lib.spicy_policy_workspace_bytes(1000, 4) == 256 + 8192 + 32000
    assert lib.spicy_policy_workspace_bytes(-1, 4) == 0
    P = 0x1000

    def call(k=P, v=P, total=100, H=4, d=128, dtype=1, so=P, B=2, pp=P, pi=P, R=16, nnz=40, N=5, L=3, sink=0,
             recent=0, seg=P, ssp=P, mask=P, ws=P, wsb=1 << 30):
        return lib.spicy_policy(k, v, total, H, d, dtype, so, B, pp, pi, R, nnz, N, L, sink, recent, seg, ssp,
                                mask, ws, wsb, None)

    assert call(k=0) == 1
    assert call(mask=0) == 1
    assert call(pi=0) == 1
    assert call(N=0) == 1
    assert call(R=0) == 1
    assert call(R=17) == 1
    assert call(L=-1) == 1
    assert call(sink=-1) == 1
    assert call(B=-1) == 1
    assert call(total=-5) == 1
    assert call(B=1 << 20, N=1 << 12) == 1  # B * N + 1 overflows int32
    assert call(dtype=0) == 4               # fp32 inputs: not supported by the policy
    assert call(dtype=7) == 1
    assert call(d=96) == 4
    assert call(H=17) == 4
    assert call(wsb=100) == 3
    assert call(B=0) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(cgd, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(cgd, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        cgd.load_library()
