"""Test-side fp64 versions of the streaming algorithms the pages describe.

These are independent of the oracle (which is the plain three-pass
definition): they follow the streaming/tiled forms, so agreement between the
two pins the oracle to a second formulation, not to itself.

  * online_stats:  element-by-element recurrence of running max m and running
    denominator l ('Online Softmax -- the mathematical heart of
    FlashAttention' section 2; 'Online softmax in attention -- why and how',
    section "The online formulation"), skipping while nothing finite has been
    seen ('Online Softmax & FlashAttention', Step 1).
  * tile_stats:    the same promoted to tiles with a tile-local max and sum
    (first page, section 4).
  * merge_ml:      the associative (m, l) merge with the guard for two -inf
    sides ('Online Softmax & FlashAttention', Step 1).
  * flash_v1:      KV-block outer loop, Q-block inner loop, normalised O that is
    re-scaled and divided at every block ('Online Softmax & FlashAttention',
    Step 2).
  * flash_v2:      Q-block outer loop, unnormalised (m, l, o) state per row,
    one division at the end, LSE returned (its Step 3; first page section 5).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


def online_stats(x, trace=False):
    m, l = NEG_INF, 0.0
    ms, ls = [], []
    for xi in x:
        m_new = max(m, xi)
        if m_new == NEG_INF:        # nothing finite yet
            ms.append(m)
            ls.append(l)
            continue
        l = l * math.exp(m - m_new) + math.exp(xi - m_new)
        m = m_new
        ms.append(m)
        ls.append(l)
    return (m, l, ms, ls) if trace else (m, l)


def chunk_stats(c):
    """(tile max, tile sum of exp(x - tile max)); (-inf, 0) for an all-masked tile."""
    c = np.asarray(c, dtype=np.float64)
    if c.size == 0:
        return NEG_INF, 0.0
    m = float(c.max())
    if m == NEG_INF:
        return NEG_INF, 0.0
    return m, float(np.exp(c - m).sum())


def merge_ml(m1, l1, m2, l2):
    m = max(m1, m2)
    safe = 0.0 if m == NEG_INF else m
    return m, l1 * math.exp(m1 - safe) + l2 * math.exp(m2 - safe)


def merge_ml_unguarded(m1, l1, m2, l2):
    m = max(m1, m2)
    with np.errstate(invalid="ignore"):
        return m, float(np.float64(l1) * np.exp(np.float64(m1) - m)
                        + np.float64(l2) * np.exp(np.float64(m2) - m))


def tile_stats(x, widths):
    """Tile recurrence over consecutive tiles of the given widths."""
    m, l = NEG_INF, 0.0
    pos = 0
    for w in widths:
        mt, lt = chunk_stats(x[pos:pos + w])
        m, l = merge_ml(m, l, mt, lt)
        pos += w
    return m, l


def lse_of(m, l):
    return m + math.log(l) if l > 0 else NEG_INF


def _visible(N, Nk, causal, kl):
    vis = np.ones((N, Nk), dtype=bool)
    if kl is not None:
        vis[:, min(max(kl, 0), Nk):] = False
    if causal:
        i = np.arange(N)[:, None]
        j = np.arange(Nk)[None, :]
        vis &= j <= i + (Nk - N)
    return vis


def flash_v1(q, k, v, Br=4, Bc=3, scale=None, causal=False, kl=None):
    """One head: q [N,d], k/v [Nk,d] fp64.  Returns (O, LSE)."""
    N, d = q.shape
    Nk = k.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    vis = _visible(N, Nk, causal, kl)
    O = np.zeros((N, d))
    l = np.zeros(N)
    m = np.full(N, NEG_INF)
    for j0 in range(0, Nk, Bc):                   # outer: one KV block
        Kj, Vj = k[j0:j0 + Bc], v[j0:j0 + Bc]
        for i0 in range(0, N, Br):                # inner: every Q block
            S = q[i0:i0 + Br] @ Kj.T * scale
            S = np.where(vis[i0:i0 + Br, j0:j0 + Bc], S, NEG_INF)
            for r in range(S.shape[0]):
                i = i0 + r
                m_ij, l_ij = chunk_stats(S[r])
                if m_ij == NEG_INF:
                    continue
                P = np.exp(S[r] - m_ij)
                m_new, l_new = merge_ml(m[i], l[i], m_ij, l_ij)
                a_old = l[i] * math.exp(m[i] - m_new) if l[i] > 0 else 0.0
                O[i] = (a_old * O[i] + math.exp(m_ij - m_new) * (P @ Vj)) / l_new
                m[i], l[i] = m_new, l_new
    lse = np.array([lse_of(m[i], l[i]) for i in range(N)])
    return O, lse


def flash_v2(q, k, v, Br=4, Bc=3, scale=None, causal=False, kl=None):
    """One head, Q-block outer / KV inner, unnormalised o, one divide at the end."""
    N, d = q.shape
    Nk = k.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    vis = _visible(N, Nk, causal, kl)
    O = np.zeros((N, d))
    LSE = np.full(N, NEG_INF)
    for i0 in range(0, N, Br):
        rows = range(i0, min(i0 + Br, N))
        m = {i: NEG_INF for i in rows}
        l = {i: 0.0 for i in rows}
        o = {i: np.zeros(d) for i in rows}
        for j0 in range(0, Nk, Bc):
            Kj, Vj = k[j0:j0 + Bc], v[j0:j0 + Bc]
            for i in rows:
                s = (Kj @ q[i]) * scale
                s = np.where(vis[i, j0:j0 + Bc], s, NEG_INF)
                m_new = max(m[i], float(s.max()))
                if m_new == NEG_INF:
                    continue
                alpha = math.exp(m[i] - m_new)
                beta = np.exp(s - m_new)
                l[i] = alpha * l[i] + beta.sum()
                o[i] = alpha * o[i] + beta @ Vj
                m[i] = m_new
        for i in rows:
            if l[i] > 0:
                O[i] = o[i] / l[i]
                LSE[i] = m[i] + math.log(l[i])
    return O, LSE


def read_golden(path):
    """key -> list of tokens, from a '#'-commented whitespace fixture."""
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out.setdefault(key, []).append(vals)
    return out
