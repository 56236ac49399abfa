"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Bars (written here, per quantity):
  * coarsen, integer and layout data (lengths, entry kind, mass, pos_sum):
    bit-exact; alpha = bf16(ln m): bit-exact; values of exact C-points: bit
    copies; mean keys/values/beta: within 1 unit in the last place of the
    storage type (both sides accumulate in double precision and round once;
    only the last bits of sin/cos/pow may differ).
  * decode, bf16 storage: O max-abs <= 1e-2, LSE relative <= 1e-3 (bf16
    storage, fp32 accumulation).  fp32 storage: O max-abs <= 2e-5, LSE
    relative <= 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from coarse_grained_decode_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import coarse_grained_decode_amd as cgd
    cgd.load_library()


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def bf16_key(bits: np.ndarray) -> np.ndarray:
    """Monotone integer key of bf16 bit patterns (ulp distance = key difference)."""
    b = bits.astype(np.int32) & 0xFFFF
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def f32_key(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def ulp_dist(a: np.ndarray, b: np.ndarray, store: str) -> np.ndarray:
    if store == "bf16":
        return np.abs(bf16_key(a) - bf16_key(b))
    return np.abs(f32_key(a) - f32_key(b))


def touched_pages(page_table: np.ndarray, lengths: np.ndarray) -> np.ndarray:
    pages = set()
    for b, L in enumerate(lengths):
        n = -(-int(L) // 16)
        pages.update(int(p) for p in page_table[b, :n])
    return np.array(sorted(pages), dtype=np.int64)


def compare_cache(dw, ref: oracle.Cache, lengths: np.ndarray):
    """Compare the GPU cache with the oracle cache over every written page."""
    store = dw.wl.dtype
    pages = touched_pages(dw.wl.page_table, lengths)
    gk, gv, gab = host(dw.cache.k)[pages], host(dw.cache.v)[pages], host(dw.cache.ab)[pages]
    gm = host(dw.cache.meta)[pages]
    rk, rv, rab, rm = ref.k[pages], ref.v[pages], ref.ab[pages], ref.meta[pages]
    # integer layout: bit-exact
    assert np.array_equal(gm[..., 0], rm["kind"]), "entry kinds differ"
    assert np.array_equal(gm[..., 1], rm["mass"]), "masses differ"
    pos = gm[..., 2].astype(np.int64) & 0xFFFFFFFF | (gm[..., 3].astype(np.int64) << 32)
    assert np.array_equal(pos, rm["pos_sum"]), "position sums differ"
    # alpha bit-exact, beta within 1 ulp
    assert np.array_equal(gab[..., 0], rab[..., 0]), "alpha differs"
    assert ulp_dist(gab[..., 1], rab[..., 1], store).max() <= 1, "beta differs by > 1 ulp"
    # values: C-points are bit copies; macro-node means within 1 ulp
    kind = rm["kind"]
    cpt = (kind == 1)
    vt, rvt = oracle.rows(gv), oracle.rows(rv)      # [P, H, 16, d]
    assert np.array_equal(vt[cpt], rvt[cpt]), "C-point values are not exact copies"
    assert ulp_dist(vt, rvt, store).max() <= 1, "values differ by > 1 ulp"
    dk = ulp_dist(gk, rk, store)
    assert dk.max() <= 1, f"keys differ by {dk.max()} ulp"
    return dict(k_exact=float((dk == 0).mean()), v_exact=float((ulp_dist(vt, rvt, store) == 0).mean()))


def compare_decode(o, lse, ro, rlse, store):
    o = o.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), fin), "LSE finiteness differs"
    assert np.all(lse[~fin] == -np.inf) and not o[~fin].any()
    err_o = float(np.abs(o - ro).max()) if o.size else 0.0
    rel = np.abs(lse[fin] - rlse[fin]) / np.maximum(np.abs(rlse[fin]), 1.0)
    err_l = float(rel.max()) if rel.size else 0.0
    tol_o, tol_l = (1e-2, 1e-3) if store == "bf16" else (2e-5, 1e-5)
    assert err_o <= tol_o, f"O max-abs error {err_o}"
    assert err_l <= tol_l, f"LSE relative error {err_l}"
    return err_o, err_l


def upload(ref: oracle.Cache, device=DEV):
    import coarse_grained_decode_amd as cgd
    def t(a):
        if ref.store == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).to(device)
    return cgd.PagedCache(t(ref.k), t(ref.v), t(ref.ab), None)


def gpu_decode(cache, wl, lengths, num_splits=0, q=None, table=None):
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd.runner import _tensor
    qd = _tensor(wl.q if q is None else q, wl.dtype, DEV)
    tb = torch.from_numpy(np.ascontiguousarray(wl.page_table if table is None else table, dtype=np.int32)).to(DEV)
    ln = torch.from_numpy(np.ascontiguousarray(lengths, dtype=np.int32)).to(DEV)
    B, H_q, d = wl.B, wl.H_q, wl.d
    o = torch.empty(B, H_q, d, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=DEV)
    ws = cgd.workspace(cgd.spicy_decode_workspace_bytes(B, H_q, wl.H_kv, d, tb.shape[1], num_splits), DEV)
    cgd.spicy_decode_attn(cache, qd, tb, ln, o, lse, ws, num_splits)
    torch.cuda.synchronize()
    assert cgd.device_error(ws) == 0
    return o, lse


# --------------------------------------------------------------------------
# workloads (scaled where the oracle needs it; full size otherwise)
# --------------------------------------------------------------------------

CASES = {
    "tiny_fp32": lambda: W.tiny_fp32(),
    "qwen2_1.5b_layer": lambda: W.qwen2_1p5b(),
    "qwen2_7b_small": lambda: W.qwen2_7b(B=3, T=6000),
    "long_ragged_small": lambda: W.long_ragged(T_range=(9000, 20000), B=3),
    "shared_prefix_small": lambda: W.shared_prefix(B=5, prefix_T=6000, chunk_T=2000,
                                                   suffix_range=(37, 300)),
}

_cache = {}


def run_case(name):
    if name in _cache:
        return _cache[name]
    from coarse_grained_decode_amd.runner import DeviceWorkload
    wl = CASES[name]() if name in CASES else FULL[name]()
    print(f"[case] {name}: B={wl.B} H_q={wl.H_q} H_kv={wl.H_kv} d={wl.d} pages={wl.num_pages}", flush=True)
    ref_cache, ref_len, ro, rlse = oracle.run_workload(wl)
    dw = DeviceWorkload.of(wl, DEV)
    dw.run_setup()
    dw.step_once()
    torch.cuda.synchronize()
    for c in dw.setup + ([dw.step] if dw.step else []):
        assert int(c.ws[0].item()) == 0, "device error word set"
    _cache[name] = (wl, dw, ref_cache, ref_len, ro, rlse)
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
def test_coarsen_layout_matches_oracle(name):
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case(name)
    assert np.array_equal(dw.lengths.cpu().numpy(), ref_len)
    stats = compare_cache(dw, ref_cache, ref_len)
    print(f"[{name}] exact keys {stats['k_exact']:.6f} exact values {stats['v_exact']:.6f}")
    assert stats["k_exact"] > 0.999 and stats["v_exact"] > 0.999


@pytest.mark.parametrize("name", ["tiny_fp32", "qwen2_7b_small", "shared_prefix_small"])
def test_coarsen_reads_nothing_past_its_inputs(name):
    """k_pre, v and the mask sit at the front of allocations whose tail holds
    NaN (keys, values) and 0 (mask: unprotected), so the batch's last segment
    ends right before bytes that would poison any macro-node reading them (a
    read past a segment's end); the cache must still match the oracle's."""
    _need_gpu()
    from coarse_grained_decode_amd.runner import DeviceWorkload
    wl = CASES[name]()
    ref_cache, ref_len, _, _ = oracle.run_workload(wl)
    dw = DeviceWorkload.of(wl, DEV)
    pad = 64
    for c in dw.setup + ([dw.step] if dw.step else []):
        T = c.k.shape[0]
        for attr in ("k", "v"):
            t = getattr(c, attr)
            big = torch.full((T + pad,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype, device=DEV)
            big[:T] = t
            setattr(c, attr, big[:T])
        big = torch.zeros((T + pad,) + tuple(c.mask.shape[1:]), dtype=c.mask.dtype, device=DEV)
        big[:T] = c.mask
        c.mask = big[:T]
    dw.run_setup()
    dw.run_step_coarsen()
    torch.cuda.synchronize()
    for c in dw.setup + ([dw.step] if dw.step else []):
        assert int(c.ws[0].item()) == 0, "device error word set"
    assert np.array_equal(dw.lengths.cpu().numpy(), ref_len)
    compare_cache(dw, ref_cache, ref_len)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_end_to_end_matches_oracle(name):
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case(name)
    e_o, e_l = compare_decode(dw.o, dw.lse, ro, rlse, wl.dtype)
    print(f"[{name}] O max-abs {e_o:.3e}  LSE rel {e_l:.3e}")


@pytest.mark.parametrize("name", list(CASES))
def test_decode_on_oracle_cache(name):
    """Decode alone: the oracle's cache uploaded, the GPU decodes it."""
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case(name)
    o, lse = gpu_decode(upload(ref_cache), wl, ref_len)
    compare_decode(o, lse, ro, rlse, wl.dtype)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
def test_split_count_does_not_matter(splits):
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case("qwen2_7b_small")
    o, lse = gpu_decode(dw.cache, wl, ref_len, num_splits=splits)
    compare_decode(o, lse, ro, rlse, wl.dtype)


def test_page_permutation_is_bit_identical():
    """Moving pages to other physical slots (same table contents relative to
    the data) gives bit-identical O and LSE."""
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case("long_ragged_small")
    import coarse_grained_decode_amd as cgd
    perm = torch.from_numpy(np.random.default_rng(5).permutation(wl.num_pages)).to(DEV)
    k2 = torch.empty_like(dw.cache.k); k2[perm] = dw.cache.k
    v2 = torch.empty_like(dw.cache.v); v2[perm] = dw.cache.v
    a2 = torch.empty_like(dw.cache.ab); a2[perm] = dw.cache.ab
    table2 = perm.cpu().numpy()[np.maximum(wl.page_table, 0)]
    table2[wl.page_table < 0] = -1
    o1, l1 = gpu_decode(dw.cache, wl, ref_len)
    o2, l2 = gpu_decode(cgd.PagedCache(k2, v2, a2, None), wl, ref_len, table=table2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_alpha_shift_and_empty_sequences():
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case("qwen2_1.5b_layer")
    shifted = oracle.Cache(ref_cache.store, ref_cache.num_pages, ref_cache.H_kv, ref_cache.d)
    shifted.k[:] = ref_cache.k; shifted.v[:] = ref_cache.v; shifted.ab[:] = ref_cache.ab
    a = W.bf16_bits_to_f32(shifted.ab[..., 0])
    fin = np.isfinite(a)
    a[fin] += 2.0                                           # exact in bf16 for |alpha| < 64
    shifted.ab[..., 0] = W.f32_to_bf16_bits(a)
    o, lse = gpu_decode(upload(shifted), wl, ref_len)
    compare_decode(o, lse - 2.0, ro, rlse, wl.dtype)
    lens = ref_len.copy(); lens[::2] = 0
    o, lse = gpu_decode(dw.cache, wl, lens)
    lse = lse.cpu().numpy(); o = o.cpu().numpy()
    assert np.all(lse[::2] == -np.inf) and not o[::2].any()
    assert np.all(np.isfinite(lse[1::2]))


def test_repeat_runs_are_bitwise_deterministic():
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case("shared_prefix_small")
    k0 = dw.cache.k.clone(); v0 = dw.cache.v.clone(); o0 = dw.o.clone()
    dw.step_once()
    torch.cuda.synchronize()
    assert torch.equal(k0, dw.cache.k) and torch.equal(v0, dw.cache.v) and torch.equal(o0, dw.o)


RANDOM_SHAPES = [
    # (dtype, d, H_kv, G, T, landmark frac)
    ("bf16", 128, 1, 1, 100, 0.05),
    ("bf16", 128, 3, 16, 777, 0.02),
    ("bf16", 64, 2, 5, 333, 0.03),
    ("bf16", 64, 5, 8, 1500, 0.01),
    ("f32", 128, 2, 3, 500, 0.02),
    ("f32", 64, 1, 4, 65, 0.1),
    # the most KV heads the library takes (16): several workgroups per
    # segment row in the coarsening, 16 heads in every mask row
    ("bf16", 128, 16, 2, 400, 0.03),
    ("f32", 64, 16, 1, 200, 0.05),
]


@pytest.mark.parametrize("shape", RANDOM_SHAPES)
def test_random_small_shapes(shape):
    _need_gpu()
    dtype, d, H, G, T, frac = shape
    from coarse_grained_decode_amd.runner import DeviceWorkload
    wl = W.make_single(7, dtype=dtype, B=3, H_q=H * G, H_kv=H, d=d, rope_base=1e4,
                       T=[T, T // 2 + 3, 17], run=None, mean_run=9.0, frac=frac, ratio=None, grid=7,
                       permute=True, name="random")
    ref_cache, ref_len, ro, rlse = oracle.run_workload(wl)
    dw = DeviceWorkload.of(wl, DEV)
    dw.run_setup()
    dw.decode()
    torch.cuda.synchronize()
    assert np.array_equal(dw.lengths.cpu().numpy(), ref_len)
    compare_cache(dw, ref_cache, ref_len)
    compare_decode(dw.o, dw.lse, ro, rlse, dtype)


FULL = {
    "qwen2_7b_layer": W.qwen2_7b,
    "long_ragged": W.long_ragged,
    "shared_prefix": W.shared_prefix,
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_against_oracle(name):
    """The full-size workloads, in the launch configuration the benchmark times
    (automatic split count), against the oracle run on the whole workload."""
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case(name)
    assert np.array_equal(dw.lengths.cpu().numpy(), ref_len)
    stats = compare_cache(dw, ref_cache, ref_len)
    e_o, e_l = compare_decode(dw.o, dw.lse, ro, rlse, wl.dtype)
    print(f"[{name}] exact keys {stats['k_exact']:.6f}; O max-abs {e_o:.3e}  LSE rel {e_l:.3e}")
    _cache.pop(name, None)


# --------------------------------------------------------------------------
# shared-prefix decode (spicy_decode_attn_shared)
# --------------------------------------------------------------------------

SPICY_DEVERR_SHARED = 0x10


def upload_case(c):
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd.runner import _tensor
    return (cgd.PagedCache(_tensor(c.k, c.dtype, DEV), _tensor(c.v, c.dtype, DEV), _tensor(c.ab, c.dtype, DEV),
                           None), _tensor(c.q, c.dtype, DEV))


def oracle_case(c, table=None, lengths=None):
    cache = oracle.Cache(c.dtype, c.k.shape[0], c.H_kv, c.d, fill=False)
    cache.k[:] = c.k; cache.v[:] = c.v; cache.ab[:] = c.ab
    return oracle.decode(c.q, c.dtype, cache, c.H_q, c.page_table if table is None else table,
                         c.lengths if lengths is None else lengths)


def gpu_decode_shared(cache, q, table, lengths, P, H_kv, num_splits=0, expect_err=0):
    import coarse_grained_decode_amd as cgd
    B, H_q, d = q.shape
    tb = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(DEV)
    ln = torch.from_numpy(np.ascontiguousarray(lengths, dtype=np.int32)).to(DEV)
    o = torch.empty(B, H_q, d, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, H_q, dtype=torch.float32, device=DEV)
    ws = cgd.workspace(cgd.spicy_decode_shared_workspace_bytes(B, H_q, H_kv, d, tb.shape[1], P, num_splits), DEV)
    cgd.spicy_decode_attn_shared(cache, q, tb, ln, P, o, lse, ws, num_splits)
    torch.cuda.synchronize()
    assert cgd.device_error(ws) == expect_err
    return o, lse


SHARED_CASES = [
    # (seed, B, H_q, H_kv, d, dtype, prefix pages, private pages)
    (1, 7, 28, 4, 128, "bf16", 9, (1, 6)),       # 49 rows per KV head: 4 tiles, ragged last
    (2, 1, 2, 1, 64, "bf16", 5, (0, 0)),         # one sequence, prefix only
    (3, 40, 16, 1, 64, "bf16", 70, (2, 30)),     # 2 chunks of <= 64 pages, 40 tiles
    (4, 3, 6, 3, 128, "bf16", 1, (1, 3)),        # one shared page
    (5, 5, 4, 2, 64, "f32", 4, (1, 4)),          # fp32: prefix read per sequence
]


@pytest.mark.parametrize("case", SHARED_CASES)
def test_shared_prefix_decode_matches_oracle(case):
    _need_gpu()
    seed, B, H_q, H_kv, d, dtype, P, priv = case
    c = W.random_decode_case(seed, B=B, H_q=H_q, H_kv=H_kv, d=d, dtype=dtype, prefix_pages=P,
                             private_pages=priv)
    ro, rlse = oracle_case(c)
    cache, q = upload_case(c)
    for ns in (0, 1, 3):
        o, lse = gpu_decode_shared(cache, q, c.page_table, c.lengths, P, H_kv, num_splits=ns)
        compare_decode(o, lse, ro, rlse, dtype)
    # any declared prefix length up to the real one is valid
    for p in (0, P // 2, P):
        o, lse = gpu_decode_shared(cache, q, c.page_table, c.lengths, p, H_kv)
        compare_decode(o, lse, ro, rlse, dtype)


def test_shared_prefix_short_and_empty_sequences():
    """Sequences shorter than the shared prefix (and empty ones) mask the
    prefix entries past their length; the shared pages stay as they are."""
    _need_gpu()
    c = W.random_decode_case(11, B=9, H_q=14, H_kv=2, d=128, prefix_pages=12, private_pages=(1, 3))
    lengths = c.lengths.copy()
    lengths[0] = 0
    lengths[2] = 1
    lengths[3] = 5 * 16 + 7
    lengths[5] = 12 * 16
    ro, rlse = oracle_case(c, lengths=lengths)
    cache, q = upload_case(c)
    o, lse = gpu_decode_shared(cache, q, c.page_table, lengths, 12, 2)
    compare_decode(o, lse, ro, rlse, "bf16")
    assert np.all(lse.cpu().numpy()[0] == -np.inf)


def test_shared_prefix_mismatch_sets_error_bit():
    """A row whose declared prefix differs from row 0 sets the sticky
    SPICY_DEVERR_SHARED bit; the prefix is then read from row 0's ids."""
    _need_gpu()
    c = W.random_decode_case(12, B=4, H_q=8, H_kv=2, d=64, prefix_pages=6, private_pages=(2, 2))
    bad = c.page_table.copy()
    bad[2, 3] = c.page_table[1, 7]                 # another sequence's private page
    ro, rlse = oracle_case(c)                      # row 0's ids everywhere
    cache, q = upload_case(c)
    o, lse = gpu_decode_shared(cache, q, bad, c.lengths, 6, 2, expect_err=SPICY_DEVERR_SHARED)
    compare_decode(o, lse, ro, rlse, "bf16")


def test_shared_prefix_large_batch_two_dimensional_grid():
    """9000 sequences x 4 KV heads x 6 splits: more than 65536 workgroups,
    so the launch folds them into a 2-D grid; 1125 prefix tiles."""
    _need_gpu()
    c = W.random_decode_case(13, B=9000, H_q=8, H_kv=4, d=64, prefix_pages=3, private_pages=(1, 6))
    ro, rlse = oracle_case(c)
    cache, q = upload_case(c)
    o, lse = gpu_decode_shared(cache, q, c.page_table, c.lengths, 3, 4, num_splits=16)
    compare_decode(o, lse, ro, rlse, "bf16")


def test_shared_and_plain_decode_agree_on_full_workload():
    """The benchmark's shared-prefix batch decoded both ways: every page per
    sequence (spicy_decode_attn) and the prefix once (spicy_decode_attn_shared)."""
    _need_gpu()
    wl, dw, ref_cache, ref_len, ro, rlse = run_case("shared_prefix_small")
    assert dw.shared_prefix_pages > 0
    o1, l1 = gpu_decode(dw.cache, wl, ref_len)
    compare_decode(o1, l1, ro, rlse, wl.dtype)
    e = float((o1 - dw.o).abs().max())
    assert e <= 1e-2, e


def test_many_segments_run_without_hints():
    """More (segment, head) pairs than the library's destination-hint array
    holds (2^17): every macro-node takes the staged path.  Layout and decode
    as the oracle's, at the same bars as the other cases."""
    _need_gpu()
    from coarse_grained_decode_amd.runner import DeviceWorkload
    wl = W.make_single(8, dtype="bf16", B=2, H_q=16, H_kv=16, d=64, rope_base=1e4, T=[8300, 8300], run=None,
                       mean_run=9.0, frac=0.1, ratio=None, grid=2, permute=True, name="many_segments")
    call = wl.calls[-1]
    assert (len(call.seg_offsets) - 1) * call.H_kv > 1 << 17
    print(f"[case] many_segments: {len(call.seg_offsets) - 1} segments x {call.H_kv} heads", flush=True)
    ref_cache, ref_len, ro, rlse = oracle.run_workload(wl)
    dw = DeviceWorkload.of(wl, DEV)
    dw.run_setup()
    dw.decode()
    torch.cuda.synchronize()
    for c in dw.setup:
        assert int(c.ws[0].item()) == 0, "device error word set"
    assert np.array_equal(dw.lengths.cpu().numpy(), ref_len)
    compare_cache(dw, ref_cache, ref_len)
    compare_decode(dw.o, dw.lse, ro, rlse, "bf16")
