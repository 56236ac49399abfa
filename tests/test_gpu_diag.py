"""GPU parity of the diagonal closure (the per-dimension variance sidecar s2)
against the CPU oracle, through the C ABI.

SPICY-KV demo page, Claim 3 lets the sub-grid variance be a diagonal vector;
with it the logit's closure term is sum_i q_i^2 s2_i / (2d).  Bars:
  * coarsening: k, v, alpha, beta and the metadata are bit-identical to the
    same call without the sidecar (the variance only adds sums); s2 within 1
    unit in the last place of the storage type, or within 1e-12 of the
    entry's trace sum_i s2_i (the GPU forms the rotated variance from
    one-pass moments, the oracle from rotated deviations, and rotation keeps
    the trace, so any cancellation is bounded by it); C-points and nulls
    store exactly 0.
  * decode: the bars of the scalar closure (bf16 storage O max-abs <= 1e-2,
    LSE relative <= 1e-3; fp32 storage 2e-5 / 1e-5).
"""
import numpy as np
import pytest
import torch

import oracle
from coarse_grained_decode_amd import workloads as W
from test_gpu_parity import CASES, DEV, _need_gpu, compare_cache, compare_decode, host, touched_pages, ulp_dist

pytestmark = pytest.mark.gpu


def store_value(bits, store):
    if store == "bf16":
        return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(bits, dtype=np.float64)


def compare_s2(g, r, kind, store):
    """g, r: [P, H, d/8, 16, 8] storage; kind [P, H, 16] from the oracle."""
    gr, rr = oracle.rows(g), oracle.rows(r)                    # [P, H, 16, d]
    exact0 = (kind == 0) | (kind == 1)
    assert not store_value(gr[exact0], store).any(), "C-point or null entry with non-zero variance"
    mac = kind == 2
    gv, rv = store_value(gr[mac], store), store_value(rr[mac], store)
    assert np.isfinite(gv).all()
    ulp = ulp_dist(gr[mac], rr[mac], store)
    trace = rv.sum(-1, keepdims=True)
    ok = (ulp <= 1) | (np.abs(gv - rv) <= 1e-12 * trace)
    assert ok.all(), f"s2 differs: max ulp {ulp.max()}, worst abs {np.abs(gv - rv).max()}"
    return float((ulp == 0).mean()) if ulp.size else 1.0


# the parity workloads, plus bf16 at d = 64 (rotary partners 4 lanes apart
# instead of 8) with and without rotation
DIAG_CASES = dict(CASES)
DIAG_CASES["bf16_d64"] = lambda: W.qwen2_1p5b(d=64, B=4, T=4096)
DIAG_CASES["bf16_d64_no_rope"] = lambda: W.qwen2_1p5b(d=64, B=3, T=3000, rope_base=0.0)

_runs = {}


def run_diag(name):
    if name in _runs:
        return _runs[name]
    from coarse_grained_decode_amd.runner import DeviceWorkload
    wl = DIAG_CASES[name]()
    print(f"[diag case] {name}: B={wl.B} H_q={wl.H_q} H_kv={wl.H_kv} d={wl.d} pages={wl.num_pages}", flush=True)
    ref = oracle.run_workload(wl, diag=True)
    out = {}
    for diag in (False, True):
        dw = DeviceWorkload.of(wl, DEV, diag=diag)
        dw.run_setup()
        dw.step_once()
        torch.cuda.synchronize()
        for c in dw.setup + ([dw.step] if dw.step else []):
            assert int(c.ws[0].item()) == 0, "device error word set"
        out[diag] = dw
    _runs[name] = (wl, out, ref)
    return _runs[name]


@pytest.mark.parametrize("name", list(DIAG_CASES))
def test_diag_coarsen_matches_oracle(name):
    _need_gpu()
    wl, out, (rcache, rlen, ro, rlse) = run_diag(name)
    dd, dn = out[True], out[False]
    assert np.array_equal(dd.lengths.cpu().numpy(), rlen)
    pages = touched_pages(wl.page_table, rlen)
    for f in ("k", "v", "ab", "meta"):
        a, b = host(getattr(dd.cache, f))[pages], host(getattr(dn.cache, f))[pages]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{f} changed by the variance sidecar"
    compare_cache(dd, rcache, rlen)
    frac = compare_s2(host(dd.cache.s2)[pages], rcache.s2[pages], rcache.meta["kind"][pages], wl.dtype)
    print(f"[{name}] s2 exact {frac:.6f}")


@pytest.mark.parametrize("name", list(DIAG_CASES))
def test_diag_decode_end_to_end_matches_oracle(name):
    _need_gpu()
    wl, out, (rcache, rlen, ro, rlse) = run_diag(name)
    e_o, e_l = compare_decode(out[True].o, out[True].lse, ro, rlse, wl.dtype)
    print(f"[{name}] O max-abs {e_o:.3e}  LSE rel {e_l:.3e}")


def upload_diag(c, s2):
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd.runner import _tensor
    return cgd.PagedCache(_tensor(c.k, c.dtype, DEV), _tensor(c.v, c.dtype, DEV), _tensor(c.ab, c.dtype, DEV),
                          None, _tensor(s2, c.dtype, DEV))


def oracle_diag_cache(c, s2):
    cache = oracle.Cache(c.dtype, c.k.shape[0], c.H_kv, c.d, fill=False, diag=True)
    cache.k[:] = c.k; cache.v[:] = c.v; cache.ab[:] = c.ab; cache.s2[:] = s2
    return cache


DECODE_CASES = [
    # (seed, B, H_q, H_kv, d, dtype, prefix pages, private pages, query tokens)
    (41, 6, 28, 4, 128, "bf16", 0, (1, 9), 1),
    (42, 5, 16, 2, 64, "bf16", 0, (2, 5), 1),
    (43, 7, 28, 4, 128, "bf16", 5, (0, 4), 1),       # shared prefix
    (44, 4, 28, 4, 128, "bf16", 3, (1, 4), 3),       # several query tokens
    (45, 3, 8, 2, 64, "f32", 0, (1, 5), 1),          # fp32 path
    (46, 3, 8, 2, 128, "f32", 2, (1, 3), 2),
]


@pytest.mark.parametrize("case", DECODE_CASES)
def test_diag_decode_on_oracle_cache(case):
    import coarse_grained_decode_amd as cgd
    _need_gpu()
    seed, B, H_q, H_kv, d, dtype, P, priv, n_q = case
    print(f"[diag decode] seed {seed}: B={B} H_q={H_q} H_kv={H_kv} d={d} {dtype} P={P} n_q={n_q}", flush=True)
    c = W.random_decode_case(seed, B=B, H_q=H_q, H_kv=H_kv, d=d, dtype=dtype, prefix_pages=P,
                             private_pages=priv, q_tokens=n_q)
    s2 = W.random_variances(c, seed)
    ref = oracle_diag_cache(c, s2)
    if n_q == 1:
        ro, rlse = oracle.decode(c.q, c.dtype, ref, c.H_q, c.page_table, c.lengths)
    else:
        ro, rlse = oracle.decode_multi(c.q, c.dtype, ref, c.page_table, c.lengths)
    cache = upload_diag(c, s2)
    from coarse_grained_decode_amd.runner import _tensor
    q = _tensor(c.q, c.dtype, DEV)
    qm = q if n_q > 1 else q[:, None]
    tb = torch.from_numpy(c.page_table).to(DEV)
    ln = torch.from_numpy(c.lengths).to(DEV)
    Pd = P if dtype == "bf16" else 0
    for ns in (0, 1, 3):
        o = torch.empty(B, n_q, H_q, d, dtype=torch.float32, device=DEV)
        lse = torch.empty(B, n_q, H_q, dtype=torch.float32, device=DEV)
        ws = cgd.workspace(cgd.spicy_decode_multi_workspace_bytes(B, n_q, H_q, H_kv, d, tb.shape[1], Pd, ns), DEV)
        cgd.spicy_decode_attn_multi(cache, qm.contiguous(), tb, ln, Pd, o, lse, ws, ns)
        torch.cuda.synchronize()
        assert cgd.device_error(ws) == 0
        compare_decode(o.reshape(B * n_q, H_q, d), lse.reshape(B * n_q, H_q),
                       ro.reshape(B * n_q, H_q, d), rlse.reshape(B * n_q, H_q), dtype)


def test_diag_constant_variance_is_the_scalar_closure():
    """s2_i = 2 d beta for every i gives sum_i q_i^2 s2_i / (2d) = |q|^2 beta:
    the diagonal decode equals the scalar one (to the bars)."""
    import coarse_grained_decode_amd as cgd
    _need_gpu()
    B, H_q, H_kv, d = 5, 28, 4, 128
    c = W.random_decode_case(47, B=B, H_q=H_q, H_kv=H_kv, d=d, prefix_pages=0, private_pages=(2, 6))
    beta_bits = c.ab[..., 1]
    beta = store_value(beta_bits, "bf16")                         # [P, H, 16]
    s2 = np.repeat((2.0 * d * beta)[..., None], d, axis=-1)       # exact in bf16: a power-of-two multiple
    s2_store = W._store(W.chunked(s2.astype(np.float32)), "bf16")
    from test_gpu_parity import gpu_decode_shared, upload_case
    plain, q = upload_case(c)
    o1, l1 = gpu_decode_shared(plain, q, c.page_table, c.lengths, 0, H_kv)
    diag = upload_diag(c, s2_store)
    o2, l2 = gpu_decode_shared(diag, q, c.page_table, c.lengths, 0, H_kv)
    ro, rlse = oracle.decode(c.q, c.dtype, oracle_diag_cache(c, s2_store), c.H_q, c.page_table, c.lengths)
    compare_decode(o1, l1, ro, rlse, "bf16")
    compare_decode(o2, l2, ro, rlse, "bf16")
