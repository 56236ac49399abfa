"""The synthetic workloads: determinism, the policy rules, and the numbers the
pages print (tests/golden/page_numbers.txt)."""
import math
import os

import numpy as np
import pytest

import oracle
from coarse_grained_decode_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.txt")


def golden():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            out[k] = float(v)
    return out


def test_page_numbers_are_consistent():
    """28.6x is a 3.5% budget and 50x a 2.0% budget (tokens per cache entry);
    4 bytes of sidecar per d=128 bf16 node (K and V rows) is under 0.8%."""
    g = golden()
    assert round(100 / g["ratio_a"], 1) == g["budget_a_percent"]
    assert round(100 / g["ratio_b"], 1) == g["budget_b_percent"]
    d = 128
    overhead = 100 * g["sidecar_bytes"] / (2 * d * 2)
    assert overhead < g["sidecar_overhead_below_percent"]
    assert W.SINK == g["sink"] and W.RECENT == g["recent"]


@pytest.mark.parametrize("T,ratio,frac,expect", [
    (10752, 28.6, 0.01, (32, 123, 90, 376)),      # Qwen2-1.5B layer
    (32768, 28.6, 0.01, (32, 261, 502, 1146)),    # Qwen2-7B layer: "~1146 entries per head"
    (65536, 28.6, 0.01, (32, 467, 1114, 2291)),   # shared prefix
])
def test_dyadic_plan_closed_form(T, ratio, frac, expect):
    g = golden()
    n_prot = W.SINK + W.RECENT + W.landmark_count(T, frac)
    s, n_big, n_small = W.dyadic_plan(T, ratio, n_prot)
    assert (s, n_big, n_small) == expect[:3]
    segs = W.dyadic_segments(T, ratio, n_prot)
    assert segs[0] == 0 and segs[-1] == T
    sizes = np.diff(segs)
    assert np.all(sizes[:n_big] == 2 * s) and np.all(sizes[n_big:-1] == s)
    # macro-nodes = segments with an unprotected token (all but the recent-window cells)
    recent_cells = sum(1 for a, z in zip(segs[:-1], segs[1:]) if a >= T - W.RECENT)
    entries = len(segs) - 1 - recent_cells + n_prot
    assert entries == expect[3] == round(T / ratio)
    assert abs(T / entries - g["target_ratio"]) < 0.05


def test_dyadic_50x_long_contexts():
    for T in (65536, 98304, 131072, 77777):
        n_prot = W.SINK + W.RECENT + W.landmark_count(T, 0.005)
        segs = W.dyadic_segments(T, 50.0, n_prot)
        recent_cells = sum(1 for a in segs[:-1] if a >= T - W.RECENT)
        assert len(segs) - 1 - recent_cells + n_prot == round(T / 50.0)


def test_landmarks_are_top_norms_per_head():
    rng = np.random.default_rng(0)
    T, H, d = 500, 3, 16
    k = rng.standard_normal((T, H, d))
    mask = W.protection_mask(k, 8, 48, 0.02)
    L = W.landmark_count(T, 0.02)
    assert L == 10
    for h in range(H):
        assert mask[:8, h].all() and mask[T - 48:, h].all()
        mid = np.nonzero(mask[8:T - 48, h])[0] + 8
        assert mid.size == L
        norms = np.linalg.norm(k[8:T - 48, h], axis=1)
        thresh = np.sort(norms)[::-1][L - 1]
        assert np.all(np.linalg.norm(k[mid, h], axis=1) >= thresh)


def test_equal_variation_first_crossing():
    """Boundaries are first hitting times of the thresholds j*C/N (Equal-Variation
    KV Cache page, "Mathematical statement"), brute-forced on a small trajectory,
    and the variation inside every segment stays below C/N plus one quantum."""
    rng = np.random.default_rng(1)
    for trial in range(20):
        T = int(rng.integers(5, 300))
        N = int(rng.integers(2, 40))
        q = rng.integers(0, 1000, size=T).astype(np.int64)
        q[0] = 0
        q[rng.random(T) < 0.3] = 0          # flat stretches
        segs = W.equal_variation_segments(q, N)
        C = np.cumsum(q)
        total = int(C[-1])
        # brute force of the definition
        ref = {0, T}
        for j in range(1, N):
            Qj = (j * total) // N
            t = next((t for t in range(T) if C[t] >= Qj), T)
            ref.add(t)
        assert list(segs) == sorted(ref)
        for a, z in zip(segs[:-1], segs[1:]):
            inner = int(C[z - 1] - C[a])
            assert inner <= total / N + 1


def test_equal_variation_scale_invariance():
    """Multiplying the projection by a power of two scales every quantum by the
    same factor: the boundaries do not move."""
    rng = np.random.default_rng(2)
    k = rng.standard_normal((400, 2, 8)); v = rng.standard_normal((400, 2, 8))
    P = rng.standard_normal((16, 32))
    a = W.equal_variation_segments(W.variation_quanta(k, v, P), 37)
    b = W.equal_variation_segments(W.variation_quanta(k, v, 4.0 * P), 37)
    assert np.array_equal(a, b)


def test_workloads_are_deterministic():
    a = W.qwen2_7b(B=2, T=4096)
    b = W.qwen2_7b(B=2, T=4096)
    for x, y in ((a.setup[0].k, b.setup[0].k), (a.setup[0].mask, b.setup[0].mask),
                 (a.setup[0].seg_offsets, b.setup[0].seg_offsets), (a.q, b.q)):
        assert np.array_equal(x, y)


def test_qwen2_1p5b_reaches_the_target_ratio():
    """Full-size Qwen2-1.5B-shaped layer through the oracle: 376 entries per
    sequence (10752 / 28.6), i.e. the 3.5% budget."""
    wl = W.qwen2_1p5b()
    call = wl.setup[0]
    cache = oracle.Cache("bf16", wl.num_pages, wl.H_kv, wl.d)
    lengths = oracle.coarsen(call, cache)
    assert np.all(lengths <= 376) and np.all(lengths >= 374)
    assert abs(10752 / lengths.mean() - 28.6) < 0.2


def test_shared_prefix_structure():
    wl = W.shared_prefix(B=4, prefix_T=4096, chunk_T=1024, suffix_range=(40, 70))
    prefix, suffix = wl.setup
    chunk = wl.step
    assert prefix.B == 1 and suffix.B == 4 and chunk.B == 4
    pp = prefix.max_pages
    assert np.all(wl.page_table[:, :pp] == np.arange(pp))       # shared physical pages
    assert np.all(suffix.mask == 1) and suffix.n_seg == 4      # exact tokens, one segment
    S = np.diff(suffix.seq_offsets)
    assert np.all(chunk.pos_base == 4096 + S)
    assert np.all(chunk.entry_start == pp * 16 + (-(-S // 16)) * 16)
    assert chunk.mask.sum(axis=0).tolist() == [4 * W.landmark_count(1024, 0.01)] * 4


def test_variant_inputs_are_seeded_and_shaped():
    """The next-row input generators: per-token weights (a fifth zero, every
    7th segment all zero), random variance sidecars (NaN exactly where the
    decode case planted NaN), query tokens; all deterministic."""
    wl = W.qwen2_7b(B=2, T=6000)
    call = wl.calls[-1]
    w1, w2 = W.token_weights(call, 3), W.token_weights(call, 3)
    assert w1.dtype == np.int64 and w1.shape == (call.total_tokens,)
    assert np.array_equal(w1, w2) and not np.array_equal(w1, W.token_weights(call, 4))
    assert (w1 >= 0).all() and 0.1 < (w1 == 0).mean() < 0.5
    so = np.asarray(call.seg_offsets)
    for s in range(0, len(so) - 1, 7):
        assert not w1[so[s]:so[s + 1]].any()
    c = W.random_decode_case(5, B=3, H_q=8, H_kv=2, d=64, prefix_pages=2, private_pages=(1, 3))
    s2 = W.random_variances(c, 5)
    assert s2.shape == c.k.shape and np.array_equal(s2, W.random_variances(c, 5))
    vals = (s2.astype(np.uint32) << 16).view(np.float32)
    alpha = (c.ab[..., 0].astype(np.uint32) << 16).view(np.float32)
    planted = np.isnan(oracle.rows(vals)).all(-1)
    assert np.array_equal(planted, np.isnan(alpha))
    assert (oracle.rows(vals)[~planted] >= 0).all()
    q4 = W.query_tokens(wl, 4)
    assert q4.shape == (wl.B, 4, wl.H_q, wl.d) and np.array_equal(q4, W.query_tokens(wl, 4))
