"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle (oracle/spicy_oracle.c) against a closed form, a
library routine, an invariant the pages state, or brute force on tiny inputs.
Chosen so that a plausible slip (a dropped term, a wrong sign, a transposed
pair, an off-by-one in the layout) fails at least one of them.
"""
import fractions
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from coarse_grained_decode_amd import workloads as W


# ---------------------------------------------------------------------------
# helpers building tiny coarsen calls
# ---------------------------------------------------------------------------

def make_call(k, v, mask, segs, *, base=0.0, pos_base=0, dtype="f64"):
    """One sequence, one or more heads.  k, v: [T, H, d] float64."""
    T, H, d = k.shape
    segs = np.asarray(segs, dtype=np.int64)
    return W._concat_call(dtype, H, d, base, [k], [v], [np.asarray(mask, dtype=np.uint8).reshape(T, H)],
                          [segs], [pos_base], np.arange(-(-(T + 16) // 16) + 1)[None, :], [0])


def run(call, store="f64", q=None, H_q=None):
    cache = oracle.Cache(store, int(call.page_table.max()) + 1, call.H_kv, call.d)
    lengths = oracle.coarsen(call, cache, in_dtype="f64")
    out = None
    if q is not None:
        out = oracle.decode(q, "f64", cache, H_q, call.page_table, lengths)
    return cache, lengths, out


def entry(cache, call, b, h, e):
    P = call.page_table[b, e // 16]
    s = e % 16
    return dict(k=oracle.rows(cache.k)[P, h, s].astype(np.float64), v=oracle.rows(cache.v)[P, h, s].astype(np.float64),
                alpha=float(cache.ab[P, h, s, 0]), beta=float(cache.ab[P, h, s, 1]),
                kind=int(cache.meta[P, h, s]["kind"]), mass=int(cache.meta[P, h, s]["mass"]),
                pos_sum=int(cache.meta[P, h, s]["pos_sum"]))


def sdpa(q, k, v):
    """torch's scaled_dot_product_attention in float64 on the CPU (library routine)."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, None, None, :]
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    lse = torch.logsumexp((kt[0, 0] @ qt[0, 0, 0]) / math.sqrt(k.shape[-1]), dim=0)
    return o[0, 0, 0].numpy(), float(lse)


# ---------------------------------------------------------------------------
# bfloat16 rounding (the storage step)
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch_on_binary32_values():
    """For inputs that are exact binary32 values there is a single rounding, so
    the oracle's double->bf16 rounding must agree with torch's float32->bf16."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40, -1e-45])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([oracle.bf16_round(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(ref, got)


def _nearest_bf16_exact(x: float) -> int:
    """Brute force: the two bf16 neighbours of x, compared with exact rationals."""
    f = np.float32(x)
    bits = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) >> 16
    cands = {(bits + dlt) & 0xFFFF for dlt in (-1, 0, 1, 2)}
    best = None
    X = fractions.Fraction(x)
    for c in sorted(cands):
        val = oracle.bf16_value(c)
        if not math.isfinite(val) or math.copysign(1, val) != math.copysign(1, x):
            continue
        err = abs(fractions.Fraction(val) - X)
        key = (err, c & 1)  # ties: even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_bf16_round_is_single_rounding_of_doubles():
    """Direct nearest-even rounding of a double, not via binary32: values that
    land exactly on a bf16 midpoint after a binary32 rounding must still go to
    the nearer neighbour."""
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(3000) * 7.0)
    xs += [1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -8 - 2 ** -30, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 10.968749861522683]
    for x in xs:
        assert oracle.bf16_round(x) == _nearest_bf16_exact(float(x)), x
    assert oracle.bf16_round(1 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert oracle.bf16_round(1 + 2 ** -8) == 0x3F80     # tie -> even
    assert oracle.bf16_round(1 + 3 * 2 ** -8) == 0x3F82  # tie -> even


def test_alpha_ln_m_exhaustive():
    """alpha = ln m stored in bf16 for every mass up to 131072 is the nearest
    bf16 to ln m (m = 58032 is the one case where rounding through binary32
    first would give the other neighbour)."""
    ms = np.arange(1, 131073)
    got = np.array([oracle.bf16_round(math.log(int(m))) for m in ms], dtype=np.uint16)
    via_f32 = torch.from_numpy(np.log(ms.astype(np.float64)).astype(np.float32)).to(torch.bfloat16)
    via_f32 = via_f32.view(torch.int16).numpy().astype(np.uint16)
    diff = np.nonzero(got != via_f32)[0]
    assert list(ms[diff]) == [58032]
    assert got[58031] == _nearest_bf16_exact(math.log(58032))
    for m in (1, 2, 3, 16, 48, 1000, 131072):
        assert got[m - 1] == _nearest_bf16_exact(math.log(m))


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [4, 64, 128])
def test_rope_matches_complex_multiplication(d):
    rng = np.random.default_rng(d)
    for base in (1e4, 1e6, 500.0):
        for pos in (0.0, 1.0, 17.5, 65535.5, 131071.0):
            x = rng.standard_normal(d)
            # theta_i from two pow() implementations may differ in the last bit,
            # which the position multiplies
            assert np.allclose(oracle.rope(x, pos, base), brute.rotate_complex(x, pos, base),
                               rtol=0, atol=1e-14 * max(1.0, pos))


def test_rope_group_properties():
    rng = np.random.default_rng(3)
    d, base = 64, 1e4
    x, y = rng.standard_normal(d), rng.standard_normal(d)
    assert np.array_equal(oracle.rope(x, 0.0, base), x)                     # R(0) = I
    assert np.array_equal(oracle.rope(x, 123.0, 0.0), x)                    # base <= 0: identity
    assert np.array_equal(oracle.rope(x, 123.0, -1.0), x)
    r = oracle.rope(x, 1234.25, base)
    assert abs(np.linalg.norm(r) - np.linalg.norm(x)) < 1e-12               # isometry
    assert np.allclose(oracle.rope(oracle.rope(x, 37.0, base), 55.5, base),
                       oracle.rope(x, 92.5, base), atol=1e-12)              # R(a)R(b) = R(a+b)
    s, t = 1000.0, 1037.5                                                   # relative phase
    lhs = oracle.rope(x, s, base) @ oracle.rope(y, t, base)
    rhs = x @ oracle.rope(y, t - s, base)
    assert abs(lhs - rhs) < 1e-10
    # the first pair rotates by exactly the position (theta_0 = 1)
    e0 = np.zeros(d); e0[0] = 1.0
    r = oracle.rope(e0, 0.75, base)
    assert abs(r[0] - math.cos(0.75)) < 1e-15 and abs(r[d // 2] - math.sin(0.75)) < 1e-15


# ---------------------------------------------------------------------------
# coarsening: closed forms
# ---------------------------------------------------------------------------

def test_constant_segment_exact():
    """m identical F-tokens: mean = the token, variance 0, alpha = ln m.  The
    values are short dyadic rationals (as bf16 data are), so the sums are exact."""
    d, T = 8, 12
    rng = np.random.default_rng(4)
    tok = np.round(rng.standard_normal(d) * 64) / 64
    k = np.tile(tok, (T, 1))[:, None, :]
    v = np.tile(np.round(rng.standard_normal(d) * 64) / 64, (T, 1))[:, None, :]
    call = make_call(k, v, np.zeros(T), [0, T])
    cache, lengths, _ = run(call)
    assert lengths[0] == 1
    e = entry(cache, call, 0, 0, 0)
    assert np.array_equal(e["k"], tok) and np.array_equal(e["v"], v[0, 0])
    assert e["beta"] == 0.0 and e["alpha"] == math.log(T)
    assert e["kind"] == 2 and e["mass"] == T and e["pos_sum"] == T * (T - 1) // 2


def test_two_point_variance():
    """Segment {mu + a, mu - a}: per-dimension population variance ||a||^2 / d."""
    d = 16
    rng = np.random.default_rng(5)
    mu, a = rng.standard_normal(d), rng.standard_normal(d)
    k = np.stack([mu + a, mu - a])[:, None, :]
    v = rng.standard_normal((2, 1, d))
    cache, lengths, _ = run(make_call(k, v, np.zeros(2), [0, 2]))
    e = entry(cache, make_call(k, v, np.zeros(2), [0, 2]), 0, 0, 0)
    assert abs(e["beta"] - (a @ a) / d / (2 * d)) < 1e-14
    assert np.allclose(e["k"], mu, atol=1e-15)


def test_variance_matches_numpy_var():
    """beta * 2d equals numpy.var(ddof=0) averaged over dimensions (library routine)."""
    d, T = 32, 40
    rng = np.random.default_rng(6)
    k = rng.standard_normal((T, 1, d)) * 0.7 + 2.0
    v = rng.standard_normal((T, 1, d))
    mask = np.zeros(T); mask[[3, 11, 12]] = 1
    segs = [0, 10, 25, 40]
    call = make_call(k, v, mask, segs)
    cache, lengths, _ = run(call)
    e = 0
    for a, z in zip(segs[:-1], segs[1:]):
        F = [t for t in range(a, z) if not mask[t]]
        ent = entry(cache, call, 0, 0, e)
        assert abs(ent["beta"] * 2 * d - np.var(k[F, 0], axis=0, ddof=0).mean()) < 1e-13
        assert np.allclose(ent["v"], v[F, 0].mean(axis=0), atol=1e-14)
        e += 1 + sum(mask[a:z] > 0)


def test_mass_conservation_and_order():
    """Per (sequence, head): the masses of all non-null entries add up to the
    number of tokens; C-points have mass 1 and their own position; within a
    segment the macro-node comes first, then C-points by position."""
    rng = np.random.default_rng(7)
    T, H, d = 70, 3, 8
    k = rng.standard_normal((T, H, d)); v = rng.standard_normal((T, H, d))
    mask = (rng.random((T, H)) < 0.2).astype(np.uint8)
    mask[20:30, 1] = 1            # a fully protected segment on head 1
    segs = [0, 5, 20, 30, 50, 70]
    call = make_call(k, v, mask, segs, base=1e4, pos_base=100)
    cache, lengths, _ = run(call)
    counts = []
    for h in range(H):
        masses, e = 0, 0
        for a, z in zip(segs[:-1], segs[1:]):
            nC = int(mask[a:z, h].sum())
            if z - a - nC > 0:
                ent = entry(cache, call, 0, h, e); e += 1
                assert ent["kind"] == 2 and ent["mass"] == z - a - nC
                masses += ent["mass"]
            for t in range(a, z):
                if mask[t, h]:
                    ent = entry(cache, call, 0, h, e); e += 1
                    assert ent["kind"] == 1 and ent["mass"] == 1 and ent["pos_sum"] == 100 + t
                    assert ent["alpha"] == 0.0 and ent["beta"] == 0.0
                    masses += 1
        assert masses == T
        counts.append(e)
    assert lengths[0] == max(counts)
    # null padding up to the longest head and to the page boundary
    for h in range(H):
        for e in range(counts[h], -(-lengths[0] // 16) * 16):
            ent = entry(cache, call, 0, h, e)
            assert ent["kind"] == 0 and ent["alpha"] == -math.inf and ent["beta"] == 0.0
            assert not ent["k"].any() and not ent["v"].any()


def test_oracle_matches_dense_brute_force():
    """Paged C oracle vs the dense NumPy statement on random tiny inputs."""
    rng = np.random.default_rng(8)
    for trial in range(25):
        d = int(rng.choice([4, 8]))
        H = int(rng.integers(1, 4))
        T = int(rng.integers(1, 33))
        base = float(rng.choice([0.0, 100.0, 1e4]))
        pos0 = int(rng.integers(0, 1000))
        k = rng.standard_normal((T, H, d)); v = rng.standard_normal((T, H, d))
        mask = (rng.random((T, H)) < 0.3).astype(np.uint8)
        cuts = sorted(set(rng.integers(1, T, size=int(rng.integers(0, 6))).tolist())) if T > 1 else []
        segs = [0] + cuts + [T]
        G = int(rng.integers(1, 3))
        q = rng.standard_normal((1, H * G, d))
        call = make_call(k, v, mask, segs, base=base, pos_base=pos0)
        cache, lengths, (o, lse) = run(call, q=q, H_q=H * G)
        pos = [pos0 + t for t in range(T)]
        for h in range(H):
            ents = brute.entries(k[:, h], v[:, h], mask[:, h] > 0, segs, pos, base)
            for e, ref in enumerate(ents):
                got = entry(cache, call, 0, h, e)
                for key in ("kind", "mass", "pos_sum"):
                    assert got[key] == ref[key]
                assert np.allclose(got["k"], ref["k"], atol=1e-12)
                assert np.allclose(got["v"], ref["v"], atol=1e-12)
                assert abs(got["alpha"] - ref["alpha"]) < 1e-12 and abs(got["beta"] - ref["beta"]) < 1e-12
            for g in range(G):
                ref_lse, ref_o = brute.decode(q[0, h * G + g], ents)
                assert abs(lse[0, h * G + g] - ref_lse) < 1e-10
                assert np.allclose(o[0, h * G + g], ref_o, atol=1e-10)


# ---------------------------------------------------------------------------
# decode: special cases that reduce to textbook attention
# ---------------------------------------------------------------------------

def _attention_case(T=200, d=64, base=1e4, pos0=321, seed=9):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, 1, d)); v = rng.standard_normal((T, 1, d))
    q = rng.standard_normal((1, 1, d))
    krot = np.stack([brute.rotate_complex(k[t, 0], pos0 + t, base) for t in range(T)])
    return k, v, q, krot


def test_all_protected_equals_softmax_attention():
    """mass = 1 and sigma = 0 everywhere (every token a C-point): plain softmax
    attention over the RoPE-rotated keys (torch SDPA, float64)."""
    T, d, base, pos0 = 200, 64, 1e4, 321
    k, v, q, krot = _attention_case(T, d, base, pos0)
    call = make_call(k, v, np.ones(T), [0, 50, 120, T], base=base, pos_base=pos0)
    _, lengths, (o, lse) = run(call, q=q, H_q=1)
    ref_o, ref_lse = sdpa(q[0, 0], krot, v[:, 0])
    assert lengths[0] == T
    assert np.allclose(o[0, 0], ref_o, atol=1e-12) and abs(lse[0, 0] - ref_lse) < 1e-12


def test_singleton_segments_equal_full_attention():
    """Every segment of size one, nothing protected: each token is a macro-node
    of mass 1 at its own position, so the result is full RoPE attention."""
    T, d, base, pos0 = 150, 64, 1e6, 7
    k, v, q, krot = _attention_case(T, d, base, pos0, seed=10)
    call = make_call(k, v, np.zeros(T), list(range(T + 1)), base=base, pos_base=pos0)
    _, lengths, (o, lse) = run(call, q=q, H_q=1)
    ref_o, ref_lse = sdpa(q[0, 0], krot, v[:, 0])
    assert np.allclose(o[0, 0], ref_o, atol=1e-12) and abs(lse[0, 0] - ref_lse) < 1e-12


def test_identical_tokens_merge_exactly():
    """m identical tokens (no rotation): the single macro-node with
    alpha = ln m reproduces full attention exactly (m e^s = e^(s + ln m))."""
    d = 32
    rng = np.random.default_rng(11)
    parts_k, parts_v, segs = [], [], [0]
    for m in (1, 5, 17, 3, 40):
        parts_k.append(np.tile(rng.standard_normal(d), (m, 1)))
        parts_v.append(np.tile(rng.standard_normal(d), (m, 1)))
        segs.append(segs[-1] + m)
    kk = np.concatenate(parts_k); vv = np.concatenate(parts_v)
    T = kk.shape[0]
    q = rng.standard_normal((1, 1, d))
    call = make_call(kk[:, None], vv[:, None], np.zeros(T), segs, base=0.0)
    _, lengths, (o, lse) = run(call, q=q, H_q=1)
    ref_o, ref_lse = sdpa(q[0, 0], kk, vv)
    assert lengths[0] == 5
    assert np.allclose(o[0, 0], ref_o, atol=1e-13) and abs(lse[0, 0] - ref_lse) < 1e-13


def test_variance_closure_closes_jensen_gap():
    """Keys ~ N(mu, s^2 I) inside each segment, no rotation.  The closure term
    |q|^2 sigma^2 / (2 d) is the Gaussian second cumulant of q.k/sqrt(d), so
    log(Z_closure / Z_full) -> 0 as segments grow, while dropping it leaves the
    Jensen gap -v/2 with v = |q|^2 s^2 / d (SPICY-KV demo page, simulator
    paragraph and Claim 3; SPICY-KV abstract, item (4))."""
    d, s, m, nseg, reps = 64, 0.3, 1024, 4, 60
    rng = np.random.default_rng(12)
    closure, mass_only, gaps = [], [], []
    for _ in range(reps):
        mus = rng.standard_normal((nseg, d))
        k = np.concatenate([mu + s * rng.standard_normal((m, d)) for mu in mus])
        v = rng.standard_normal((nseg * m, d))
        q = rng.standard_normal((1, 1, d))
        call = make_call(k[:, None], v[:, None], np.zeros(nseg * m), list(range(0, nseg * m + 1, m)))
        cache, lengths, (o, lse) = run(call, q=q, H_q=1)
        _, full = sdpa(q[0, 0], k, v)
        closure.append(lse[0, 0] - full)
        cache.ab[..., 1] = 0.0           # drop the variance term: mass only
        _, lse0 = oracle.decode(q, "f64", cache, 1, call.page_table, lengths)
        mass_only.append(lse0[0, 0] - full)
        gaps.append(-(q[0, 0] @ q[0, 0]) * s * s / d / 2)
    closure, mass_only, gaps = map(np.asarray, (closure, mass_only, gaps))
    se = closure.std(ddof=1) / math.sqrt(reps)
    assert abs(closure.mean()) < 4 * se + 2e-3
    resid = mass_only - gaps
    assert abs(resid.mean()) < 4 * resid.std(ddof=1) / math.sqrt(reps) + 2e-3
    assert mass_only.mean() < -0.03          # the gap is really there without the closure


# ---------------------------------------------------------------------------
# decode: invariants
# ---------------------------------------------------------------------------

def _random_cache(seed=13, T=300, H=2, G=3, d=16, base=1e4):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, H, d)); v = rng.standard_normal((T, H, d))
    mask = (rng.random((T, H)) < 0.1).astype(np.uint8)
    segs = [0] + sorted(set(rng.integers(1, T, size=40).tolist())) + [T]
    q = rng.standard_normal((1, H * G, d))
    call = make_call(k, v, mask, segs, base=base, pos_base=50)
    cache, lengths, (o, lse) = run(call, q=q, H_q=H * G)
    return call, cache, lengths, q, o, lse


def test_alpha_shift_shifts_lse():
    call, cache, lengths, q, o, lse = _random_cache()
    finite = np.isfinite(cache.ab[..., 0])
    cache.ab[..., 0][finite] += 2.5
    o2, lse2 = oracle.decode(q, "f64", cache, q.shape[1], call.page_table, lengths)
    assert np.allclose(lse2, lse + 2.5, atol=1e-12) and np.allclose(o2, o, atol=1e-12)


def test_page_permutation_and_nulls_are_invisible():
    call, cache, lengths, q, o, lse = _random_cache(seed=14)
    npg = cache.num_pages
    perm = np.random.default_rng(0).permutation(npg)
    c2 = oracle.Cache("f64", npg, cache.H_kv, cache.d)
    c2.k[perm] = cache.k; c2.v[perm] = cache.v; c2.ab[perm] = cache.ab
    table = perm[call.page_table]
    o2, lse2 = oracle.decode(q, "f64", c2, q.shape[1], table, lengths)
    assert np.array_equal(o2, o) and np.array_equal(lse2, lse)
    # extra trailing null entries change nothing
    L = int(lengths[0])
    padded = np.array([-(-L // 16) * 16])
    o3, lse3 = oracle.decode(q, "f64", cache, q.shape[1], call.page_table, padded)
    assert np.array_equal(o3, o) and np.array_equal(lse3, lse)


def test_empty_sequence():
    call, cache, lengths, q, o, lse = _random_cache(seed=15)
    o2, lse2 = oracle.decode(q, "f64", cache, q.shape[1], call.page_table, np.zeros(1, np.int32))
    assert np.all(lse2 == -np.inf) and not o2.any()


def test_storage_rounding_is_applied_once():
    """bf16 storage: every stored number is the nearest bf16 of the exact
    (float64-storage) value."""
    call, cache, lengths, q, o, lse = _random_cache(seed=16, T=64, H=1, G=1, d=8)
    c16 = oracle.Cache("bf16", cache.num_pages, 1, 8)
    oracle.coarsen(call, c16, in_dtype="f64")
    n = -(-int(lengths[0]) // 16)
    for arr64, arr16 in ((cache.k, c16.k), (cache.v, c16.v), (cache.ab, c16.ab)):
        a = arr64[:n].ravel(); b = arr16[:n].ravel()
        for x, bits in zip(a, b):
            assert oracle.bf16_round(float(x)) == int(bits)


def test_errors_are_reported():
    call, cache, lengths, q, o, lse = _random_cache(seed=17)
    bad = call.page_table.copy(); bad[0, 0] = cache.num_pages + 5
    with pytest.raises(ValueError):
        oracle.decode(q, "f64", cache, q.shape[1], bad, lengths)
    with pytest.raises(ValueError):
        oracle.decode(q, "f64", cache, q.shape[1], call.page_table[:, :1], lengths)


def test_decode_multi_is_per_token_decode():
    """Several query tokens per sequence: every token's rows attend to the
    sequence's entries as a single query does."""
    c = W.random_decode_case(40, B=3, H_q=8, H_kv=2, d=64, q_tokens=3, dtype="f32")
    cache = oracle.Cache(c.dtype, c.k.shape[0], c.H_kv, c.d, fill=False)
    cache.k[:] = c.k; cache.v[:] = c.v; cache.ab[:] = c.ab
    o, lse = oracle.decode_multi(c.q, c.dtype, cache, c.page_table, c.lengths)
    assert o.shape == (3, 3, 8, 64) and lse.shape == (3, 3, 8)
    for t in range(3):
        o1, l1 = oracle.decode(np.ascontiguousarray(c.q[:, t]), c.dtype, cache, 8, c.page_table, c.lengths)
        assert np.array_equal(o[:, t], o1) and np.array_equal(lse[:, t], l1)


def test_decode_work_items_are_the_whole_decode():
    """The decode split into (sequence, KV head) work items over threads gives
    exactly the one-thread result (each row's arithmetic is the same)."""
    c = W.random_decode_case(41, B=3, H_q=8, H_kv=2, d=64, q_tokens=1, dtype="bf16")
    cache = oracle.Cache(c.dtype, c.k.shape[0], c.H_kv, c.d, fill=False)
    cache.k[:] = c.k; cache.v[:] = c.v; cache.ab[:] = c.ab
    q = np.ascontiguousarray(c.q)                      # [B, H_q, d] with one query token
    o1, l1 = oracle.decode(q, c.dtype, cache, 8, c.page_table, c.lengths, threads=1)
    o4, l4 = oracle.decode(q, c.dtype, cache, 8, c.page_table, c.lengths, threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4)


def test_decode_rejects_misshaped_queries():
    """A query array that is not [B, H_q, d] of the stated storage is refused
    before the C code reads it (it would read past the array's end)."""
    c = W.random_decode_case(41, B=3, H_q=8, H_kv=2, d=64, dtype="bf16")
    cache = oracle.Cache(c.dtype, c.k.shape[0], c.H_kv, c.d, fill=False)
    cache.k[:] = c.k; cache.v[:] = c.v; cache.ab[:] = c.ab
    with pytest.raises(ValueError):
        oracle.decode(np.ascontiguousarray(c.q[:, 0]), c.dtype, cache, 8, c.page_table, c.lengths)
    with pytest.raises(ValueError):
        oracle.decode(c.q.astype(np.float32), c.dtype, cache, 8, c.page_table, c.lengths)
    with pytest.raises(ValueError):
        oracle.decode(c.q, c.dtype, cache, 8, c.page_table, c.lengths[:2])
