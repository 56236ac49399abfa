"""Pins of the oracle's diagonal closure (per-dimension sub-grid variance)
against things other than itself.

SPICY-KV demo page, Claim 3 names the sub-grid variance as a scalar, a
diagonal vector or low-rank; the diagonal reading stores, per macro-node, the
per-dimension population variance s2 of its member keys rotated to the
anchor (the frame of the stored key), and the logit's closure term becomes
sum_i q_i^2 s2_i / (2 d).  Pins:
  * trace: sum_i s2_i = d sigma^2 of the scalar closure (rotation keeps the
    trace), with RoPE on;
  * two points {mu +- a}: s2 = (R(tbar) a)^2, the rotation done here by
    complex multiplication; a constant segment: s2 = 0; C-points and nulls 0;
  * isotropic spread (|a_i| all equal, no rotation): the diagonal closure
    decodes exactly like the scalar one;
  * anisotropic Gaussian keys inside one segment, no rotation: against the
    exact log partition sum of every token (numpy logsumexp), the diagonal
    closure's error per query is far below the scalar closure's.
"""
import numpy as np

import oracle
from coarse_grained_decode_amd import workloads as W


def call_of(k, v, mask, segs, base=0.0, pos_base=0):
    T, H, d = k.shape
    return W._concat_call("f64", H, d, base, [k], [v], [np.asarray(mask, dtype=np.uint8).reshape(T, H)],
                          [np.asarray(segs, dtype=np.int64)], [pos_base],
                          np.arange(-(-(T + 16) // 16) + 1)[None, :], [0])


def coarsen(call, diag=True):
    cache = oracle.Cache("f64", int(call.page_table.max()) + 1, call.H_kv, call.d, diag=diag)
    lengths = oracle.coarsen(call, cache, in_dtype="f64")
    return cache, lengths


def entry_rows(cache, x):
    return oracle.rows(x)                                # [P, H, 16, d]


def test_trace_is_the_scalar_variance_with_rope():
    rng = np.random.default_rng(3)
    T, H, d = 96, 2, 32
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    mask = rng.random((T, H)) < 0.1
    segs = [0, 11, 30, 47, 60, 96]
    cache, lengths = coarsen(call_of(k, v, mask, segs, base=1e4, pos_base=1234))
    s2 = entry_rows(cache, cache.s2)
    macro = cache.meta["kind"] == 2
    assert macro.sum() > 0
    beta = cache.ab[..., 1]
    # sum_i s2_i = d sigma^2 = d * (2 d beta)
    np.testing.assert_allclose(s2[macro].sum(-1), 2.0 * d * d * beta[macro], rtol=1e-12, atol=1e-14)
    # C-points and nulls carry no variance
    assert not s2[(cache.meta["kind"] == 1) | (cache.meta["kind"] == 0)].any()


def test_two_points_give_the_rotated_spread():
    d, base = 16, 1e4
    rng = np.random.default_rng(5)
    mu, a = rng.standard_normal(d), rng.standard_normal(d)
    k = np.stack([mu + a, mu - a])[:, None, :]
    v = np.zeros_like(k)
    pos_base = 777
    cache, _ = coarsen(call_of(k, v, np.zeros((2, 1)), [0, 2], base=base, pos_base=pos_base))
    s2 = entry_rows(cache, cache.s2)[0, 0, 0]
    tbar = pos_base + 0.5
    half = d // 2
    theta = base ** (-2.0 * np.arange(half) / d)
    za = (a[:half] + 1j * a[half:]) * np.exp(1j * tbar * theta)     # half-split pairs as complex numbers
    want = np.concatenate([za.real ** 2, za.imag ** 2])
    np.testing.assert_allclose(s2, want, rtol=1e-12, atol=1e-15)
    # a constant segment has no spread (4 copies: their mean is exact)
    kc = np.tile(mu, (4, 1))[:, None, :]
    cache, _ = coarsen(call_of(kc, np.zeros_like(kc), np.zeros((4, 1)), [0, 4], base=base))
    assert not entry_rows(cache, cache.s2)[0, 0, 0].any()


def test_isotropic_spread_decodes_like_the_scalar_closure():
    rng = np.random.default_rng(8)
    T, d = 64, 16
    mu = rng.standard_normal((T // 2, d))
    signs = rng.choice([-0.4, 0.4], size=(T // 2, d))        # |a_i| equal: every s2_i the same
    k = np.empty((T, 1, d))
    k[0::2, 0] = mu + signs
    k[1::2, 0] = mu - signs
    v = rng.standard_normal((T, 1, d))
    segs = list(range(0, T + 1, 2))                            # each pair is one segment
    call = call_of(k, v, np.zeros((T, 1)), segs)
    q = rng.standard_normal((1, 3, d))
    cd, lend = coarsen(call, diag=True)
    cs, lens = coarsen(call, diag=False)
    od, ld = oracle.decode(q, "f64", cd, 3, call.page_table, lend)
    os_, ls = oracle.decode(q, "f64", cs, 3, call.page_table, lens)
    np.testing.assert_allclose(od, os_, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ld, ls, rtol=1e-13)


def test_anisotropic_gaussian_keys_diagonal_closure_is_exact_in_the_limit():
    rng = np.random.default_rng(11)
    d, m, nq = 16, 20000, 64
    sig = np.linspace(0.1, 0.9, d)                              # anisotropic spread
    mu = rng.standard_normal(d) * 0.5
    keys = mu + sig * rng.standard_normal((m, d))
    k = keys[:, None, :]
    v = np.zeros_like(k)
    call = call_of(k, v, np.zeros((m, 1)), [0, m])
    q = rng.standard_normal((1, nq, d))
    full = np.log(np.exp((q[0] @ keys.T) / np.sqrt(d)).sum(1))  # exact log partition sum over all tokens
    errs = {}
    for diag in (True, False):
        cache, lengths = coarsen(call, diag=diag)
        _, lse = oracle.decode(q, "f64", cache, nq, call.page_table, lengths)
        errs[diag] = np.abs(lse[0] - full)
    assert errs[True].mean() < 0.25 * errs[False].mean(), (errs[True].mean(), errs[False].mean())
    assert errs[True].mean() < 0.01
