"""Pins of the oracle's per-step policy (equal-variation segments, key-norm
landmarks) against things other than itself.

The policy is integer arithmetic end to end (oracle/spicy_oracle.c,
oracle_policy), so each pin is exact:
  * fix16: exhaustive over every bf16 bit pattern, against exact rational
    arithmetic (Python fractions, whose round() ties to even);
  * the integer square root: against math.isqrt;
  * the variation d_t: brute force with Python integers on tiny inputs;
  * the boundaries: N - 1 equal jumps put the breakpoints exactly at the
    jumps (Equal-Variation KV Cache page, "Mathematical statement": equal
    increments of cumulative variation); a constant trajectory has no
    variation and gives one segment; the first-hitting property
    C[b_j - 1] < Q_j <= C[b_j]; the per-segment variation bound
    C_T / N + max d_t;
  * the landmarks: numpy's lexsort on exact integer norms, ties to the lower
    position; sink and recent always kept.
"""
import fractions
import math
import random

import numpy as np
import pytest

import oracle
from coarse_grained_decode_amd import workloads as W

SAT = 1 << 28


def fix16_exact(bits: int) -> int:
    """x * 2^16 rounded half to even and clamped, from the bit pattern by
    exact rational arithmetic."""
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0xFF:
        return 0 if m else (-SAT if s else SAT)
    if e == 0:
        x = fractions.Fraction(m, 1 << 133)                # subnormal: m * 2^-133
    else:
        x = fractions.Fraction(128 + m) * fractions.Fraction(2) ** (e - 134)
    r = round(x * (1 << 16))                               # Fraction.__round__: ties to even
    r = max(-SAT, min(SAT, r))
    return -r if s else r


def test_fix16_exhaustive():
    got = np.array([oracle.fix16(b) for b in range(1 << 16)], dtype=np.int64)
    want = np.array([fix16_exact(b) for b in range(1 << 16)], dtype=np.int64)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"fix16 differs at {[hex(int(b)) for b in bad[:8]]}"


def test_isqrt_against_math():
    rng = random.Random(11)
    xs = [0, 1, 2, 3, 4, (1 << 128) - 1, (1 << 64) ** 2 - 1]
    for _ in range(3000):
        xs.append(rng.getrandbits(rng.randint(1, 128)))
        r = rng.getrandbits(64)
        xs.extend([r * r, r * r - 1 if r else 0, r * r + 1 if r * r + 1 < (1 << 128) else r * r])
    for x in xs:
        assert oracle.isqrt_u128(x) == math.isqrt(x), x


def proj_lists(rows):
    """rows: list of lists of signed 1-based column ids -> (ptr, idx)."""
    ptr = np.cumsum([0] + [len(r) for r in rows]).astype(np.int32)
    idx = np.asarray([c for r in rows for c in r], dtype=np.int32)
    return ptr, idx


def bf16(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def variation_brute(k, v, so, ptr, idx):
    """d_t from the definition with Python integers."""
    T, H, d = k.shape
    width = H * d
    out = np.zeros(T, dtype=np.int64)
    for b in range(len(so) - 1):
        prev = None
        for t in range(int(so[b]), int(so[b + 1])):
            x = [fix16_exact(int(c)) for c in k[t].reshape(-1)] + [fix16_exact(int(c)) for c in v[t].reshape(-1)]
            z = []
            for r in range(len(ptr) - 1):
                acc = 0
                for e in idx[ptr[r]:ptr[r + 1]]:
                    c = abs(int(e)) - 1
                    acc += x[c] if e > 0 else -x[c]
                z.append(acc)
            if prev is not None:
                out[t] = math.isqrt(sum((a - p) ** 2 for a, p in zip(z, prev)))
            prev = z
    return out


def test_variation_matches_brute_force():
    c = W.random_policy_case(3, B=3, T_range=(5, 40), H=2, d=8, n_segments=4, n_landmarks=2, proj_rows=5)
    r = oracle.policy(c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, 4, 2, 0, 0)
    want = variation_brute(c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx)
    assert np.array_equal(r.variation, want)
    # first token of every sequence has no predecessor
    assert not r.variation[c.seq_offsets[:-1]].any()


def test_equal_jumps_put_boundaries_at_the_jumps():
    """A trajectory that is constant except for N - 1 jumps of equal size has
    C_t = J * (jumps up to t), so the j-th threshold floor(j (N-1) J / N)
    lies in ((j - 1) J, j J] and is first reached at the j-th jump."""
    T, H, d, N = 64, 1, 8, 5
    jumps = [7, 20, 33, 50]
    col = 3                                           # k dimension 3 of head 0
    x = np.zeros(T, dtype=np.float32)
    level = 0.0
    for t in range(T):
        if t in jumps:
            level = 1.0 - level                       # alternate 0 <-> 1: |step| = 1 each time
        x[t] = level
    k = np.zeros((T, H, d), dtype=np.float32)
    k[:, 0, col] = x
    v = np.full((T, H, d), 0.5, dtype=np.float32)     # constant: no variation
    ptr, idx = proj_lists([[col + 1, 2 * d], [-(col + 1)], [5, 9], [-(col + 1), 12]])
    so = np.array([0, T], dtype=np.int32)
    r = oracle.policy(bf16(k), bf16(v), so, ptr, idx, N, 0, 0, 0)
    assert r.seg_offsets.tolist() == [0] + jumps + [T]
    d_jump = math.isqrt(3 * (1 << 32))                # three rows see column `col`
    assert sorted(set(r.variation.tolist())) == [0, d_jump]


def test_constant_trajectory_gives_one_segment():
    T, H, d, N = 40, 2, 8, 6
    k = np.tile(np.linspace(-1, 1, H * d, dtype=np.float32).reshape(1, H, d), (T, 1, 1))
    v = -k
    c = W.random_policy_case(0, B=1, T_range=(T, T), H=H, d=d, n_segments=N, n_landmarks=0)
    so = np.array([0, T], dtype=np.int32)
    r = oracle.policy(bf16(k), bf16(v), so, c.spec.proj_ptr, c.spec.proj_idx, N, 0, 0, 0)
    assert not r.variation.any()
    # every threshold is 0, first reached at token 0: N - 1 empty slots, then [0, T)
    assert r.seg_offsets.tolist() == [0] * N + [T]


@pytest.mark.parametrize("seed,N", [(1, 9), (2, 33), (4, 1), (5, 200)])
def test_first_hitting_property_and_variation_bound(seed, N):
    c = W.random_policy_case(seed, B=4, T_range=(1, 260), H=2, d=32, n_segments=N, n_landmarks=3)
    r = oracle.policy(c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, N, 3, 0, 0)
    so = c.seq_offsets
    assert r.seq_seg_ptr.tolist() == [b * N for b in range(len(so))]
    for b in range(len(so) - 1):
        t0, t1 = int(so[b]), int(so[b + 1])
        seg = r.seg_offsets[b * N: b * N + N + 1].astype(np.int64)
        assert seg[0] == t0 and seg[-1] == t1 and np.all(np.diff(seg) >= 0)
        C = np.cumsum(r.variation[t0:t1])
        CT = int(C[-1]) if t1 > t0 else 0
        dmax = int(r.variation[t0:t1].max()) if t1 > t0 else 0
        for j in range(1, N):
            Q = (j * CT) // N
            bj = int(seg[j]) - t0
            assert bj < t1 - t0 or t1 == t0
            assert C[bj] >= Q
            if bj > 0:
                assert C[bj - 1] < Q
        # variation inside a segment (between its first and last token) stays
        # within one share of the total plus one step
        for j in range(N):
            a, z = int(seg[j]) - t0, int(seg[j + 1]) - t0
            if z - a >= 2:
                assert C[z - 1] - C[a] <= CT / N + dmax


def test_landmarks_match_lexsort_with_ties():
    T, H, d = 120, 3, 16
    c = W.random_policy_case(9, B=1, T_range=(T, T), H=H, d=d, n_segments=3, n_landmarks=0)
    k = c.k.copy()
    k[40] = k[10]                                     # equal norms: the lower position must win
    k[77] = k[10]
    k[90, 1] = k[5, 1]
    sink, recent, L = 4, 6, 13
    r = oracle.policy(k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, 3, L, sink, recent)
    fk = np.vectorize(fix16_exact, otypes=[object])(k.astype(np.int64))
    for h in range(H):
        norms = np.array([sum(int(a) * int(a) for a in fk[t, h]) for t in range(T)], dtype=object)
        cand = np.arange(sink, T - recent)
        order = sorted(cand.tolist(), key=lambda t: (-norms[t], t))
        want = np.zeros(T, dtype=np.uint8)
        want[:sink] = 1
        want[T - recent:] = 1
        want[order[:L]] = 1
        assert np.array_equal(r.mask[:, h], want), h
        assert r.mask[:, h].sum() == sink + recent + L
        assert np.array_equal(r.norm2[:, h].astype(object), norms)


def test_landmarks_when_candidates_run_out():
    c = W.random_policy_case(12, B=3, T_range=(3, 12), H=2, d=8, n_segments=2, n_landmarks=50, sink=2, recent=3)
    r = oracle.policy(c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, 2, 50, 2, 3)
    assert r.mask.all()                               # every position is sink, recent or landmark
