"""Dense NumPy brute force of the same definitions — TEST INFRASTRUCTURE ONLY.

A second, structurally different statement of SPICY-KV coarsening and decode
for tiny inputs: no pages, no page tables, no padding — per (sequence, KV head)
a Python list of entries, built token by token, then the decode sum evaluated
entry by entry.  It exists to catch indexing, paging and ordering mistakes in
the C oracle (spicy_oracle.c); the mathematical pins live in the tests.

Definitions (SPICY-KV demo page, section 2 and Claims 2-3): a segment's
unprotected tokens merge into one node with mass m, mean pre-RoPE key rotated
to the mean position, mean value, alpha = ln m, beta = var/(2 d) where var is the
per-dimension population variance; protected tokens stay exact; the logit is
q.k/sqrt(d) + alpha + |q|^2 beta.
"""
from __future__ import annotations

import math

import numpy as np


def rotate_complex(x: np.ndarray, pos: float, base: float) -> np.ndarray:
    """RoPE written with complex numbers: pair (x_i, x_{i+d/2}) is the complex
    number x_i + i x_{i+d/2}, multiplied by exp(i pos theta_i),
    theta_i = base^(-2i/d).  base <= 0: identity."""
    d = x.shape[-1]
    h = d // 2
    if not base > 0:
        return np.array(x, dtype=np.float64)
    theta = np.power(float(base), -2.0 * np.arange(h) / d)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * pos * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def entries(k: np.ndarray, v: np.ndarray, mask: np.ndarray, seg_bounds, positions, base: float):
    """Entries of one (sequence, head): k, v [T, d] float64, mask [T] bool,
    seg_bounds relative offsets, positions [T].  Returns a list of dicts."""
    out = []
    d = k.shape[1]
    for a, z in zip(seg_bounds[:-1], seg_bounds[1:]):
        F = [t for t in range(a, z) if not mask[t]]
        C = [t for t in range(a, z) if mask[t]]
        if F:
            kF = k[F]
            mean = kF.mean(axis=0)
            var = float(np.var(kF, axis=0, ddof=0).mean())
            tbar = float(np.mean([positions[t] for t in F]))
            out.append(dict(k=rotate_complex(mean, tbar, base), v=v[F].mean(axis=0),
                            alpha=math.log(len(F)), beta=var / (2 * d), kind=2, mass=len(F),
                            pos_sum=int(sum(positions[t] for t in F))))
        for t in C:
            out.append(dict(k=rotate_complex(k[t], positions[t], base), v=v[t].copy(), alpha=0.0,
                            beta=0.0, kind=1, mass=1, pos_sum=int(positions[t])))
    return out


def decode(q: np.ndarray, ents) -> tuple:
    """LSE and O of one query over a list of entries, term by term."""
    d = q.shape[0]
    n2 = float(q @ q)
    s = []
    for e in ents:
        if e["alpha"] == -math.inf:
            continue
        s.append(float(q @ e["k"]) / math.sqrt(d) + e["alpha"] + n2 * e["beta"])
    if not s:
        return -math.inf, np.zeros(d)
    m = max(s)
    z = sum(math.exp(x - m) for x in s)
    lse = m + math.log(z)
    o = np.zeros(d)
    live = [e for e in ents if e["alpha"] != -math.inf]
    for x, e in zip(s, live):
        o += math.exp(x - lse) * e["v"]
    return lse, o
