"""Test-side fp64 streaming formulations of softmax and attention.

The oracle computes the plain three-pass definition.  The functions here
reach the same numbers through the streaming statistics the pages build on,
so agreement between the two pins the oracle to a second formulation rather
than to itself.  They are written from the formulas, not from any printed
program:

* A row segment is summarised by the pair (m, l): its max and the sum of
  exp(x - m) over it ('Online Softmax -- the mathematical heart of
  FlashAttention', sections 2 and 4; 'Online Softmax & FlashAttention',
  Step 1).  An empty or fully masked segment is (-inf, 0).
* Two pairs combine to (M, l1 * w1 + l2 * w2) with M = max(m1, m2) and
  w_i = exp(m_i - M), where a side that has seen nothing has weight 0 (the
  guard of Step 1, which keeps -inf - (-inf) out of the arithmetic).  The
  operation is associative, so a scan, a left fold and any tree of
  combinations agree.
* Attention over key blocks carries the pair and an output accumulator per
  query row and folds each key block in with the combination weights: the
  accumulator either stays unnormalised and is divided once at the end
  (research-hub 'Online Softmax' page, "Why it matters"; first page section
  5), or is kept normalised and re-divided after every block (the V1
  variant of Step 2).  Blocks may have any widths, and query blocks are
  independent.

Everything is vectorised with numpy over rows; the only Python loops run
over blocks or over the pairs being combined.
"""
from __future__ import annotations

import functools
import itertools

import numpy as np

NEG_INF = float("-inf")


# ----------------------------------------------------------------- (m, l) pairs
def pair_of(x):
    """Pair(s) of the segment(s) along the last axis: (max, sum exp(x - max));
    (-inf, 0) where nothing is finite.  Scalars for 1-D input."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] == 0:
        shape = x.shape[:-1]
        return np.full(shape, NEG_INF)[()], np.zeros(shape)[()]
    m = x.max(axis=-1)
    empty = np.isneginf(m)
    shift = np.where(empty, 0.0, m)
    l = np.where(empty, 0.0, np.exp(x - np.expand_dims(shift, -1)).sum(axis=-1))
    return m[()], l[()]


def combine_weights(m1, m2):
    """(M, w1, w2): the common max and each side's weight exp(m_i - M), 0 for a
    side without any finite entry."""
    m1 = np.asarray(m1, dtype=np.float64)
    m2 = np.asarray(m2, dtype=np.float64)
    M = np.maximum(m1, m2)
    with np.errstate(invalid="ignore"):
        w1 = np.where(np.isneginf(m1), 0.0, np.exp(m1 - M))
        w2 = np.where(np.isneginf(m2), 0.0, np.exp(m2 - M))
    return M[()], w1[()], w2[()]


def combine(a, b):
    """a (+) b for pairs a = (m1, l1), b = (m2, l2) (scalars or arrays)."""
    M, w1, w2 = combine_weights(a[0], b[0])
    return M, a[1] * w1 + b[1] * w2


def combine_unguarded(a, b):
    """The same formula with the weights taken as exp(m_i - M) even when both
    sides are empty (negative control: -inf - (-inf) is NaN)."""
    M = np.maximum(np.float64(a[0]), np.float64(b[0]))
    with np.errstate(invalid="ignore"):
        return M, a[1] * np.exp(np.float64(a[0]) - M) + b[1] * np.exp(np.float64(b[0]) - M)


def scan(x):
    """Single pass over a 1-D row, each element entering as the pair (x_i, 1)
    (a masked element as (-inf, 0)).  Returns the final pair and the list of
    running pairs after each element."""
    singles = [(float(v), 0.0 if v == NEG_INF else 1.0) for v in np.asarray(x, dtype=np.float64)]
    states = list(itertools.accumulate(singles, combine, initial=(NEG_INF, 0.0)))[1:]
    final = states[-1] if states else (NEG_INF, 0.0)
    return (float(final[0]), float(final[1])), [(float(m), float(l)) for m, l in states]


def segments(x, widths):
    """The pairs of consecutive segments of the given widths along the last axis."""
    edges = np.cumsum([0] + list(widths))
    return [pair_of(np.asarray(x)[..., a:b]) for a, b in zip(edges[:-1], edges[1:])]


def fold_left(pairs):
    return functools.reduce(combine, pairs, (NEG_INF, 0.0))


def fold_tree(pairs):
    """Balanced tree: combine the two halves' results (lower half first)."""
    if len(pairs) == 1:
        return pairs[0]
    h = len(pairs) // 2
    return combine(fold_tree(pairs[:h]), fold_tree(pairs[h:]))


def fold_random_tree(pairs, rng):
    """Repeatedly combine a random adjacent couple until one pair is left."""
    work = list(pairs)
    while len(work) > 1:
        i = int(rng.integers(0, len(work) - 1))
        work[i:i + 2] = [combine(work[i], work[i + 1])]
    return work[0]


def lse(pair):
    m, l = pair
    return m + np.log(l) if l > 0 else NEG_INF


# ------------------------------------------------------------------ attention
def visibility(N, Nk, causal=False, key_len=None):
    """[N, Nk] mask: key j visible to query i (key length, then the causal band
    j <= i + Nk - N)."""
    kl = Nk if key_len is None else min(max(key_len, 0), Nk)
    j = np.arange(Nk)[None, :]
    vis = np.broadcast_to(j < kl, (N, Nk))
    if causal:
        vis = vis & (j <= np.arange(N)[:, None] + (Nk - N))
    return vis


def _blocks(total, widths):
    """Half-open ranges covering [0, total): an int width repeats, a list of
    widths repeats cyclically."""
    seq = itertools.cycle([widths] if np.isscalar(widths) else list(widths))
    a = 0
    while a < total:
        b = min(total, a + int(next(seq)))
        yield a, b
        a = b


def _fold_keys(q, k, v, vis, scale, key_widths, normalised):
    """Fold every key block into the state of the query rows q (all rows at once)."""
    n, dv = q.shape[0], v.shape[1]
    m = np.full(n, NEG_INF)
    l = np.zeros(n)
    acc = np.zeros((n, dv))
    for a, b in _blocks(k.shape[0], key_widths):
        s = np.where(vis[:, a:b], (q @ k[a:b].T) * scale, NEG_INF)
        mb, lb = pair_of(s)
        mb, lb = np.atleast_1d(mb), np.atleast_1d(lb)
        ref = np.where(np.isneginf(mb), 0.0, mb)
        pv = np.exp(s - ref[:, None]) @ v[a:b]          # this block's weighted values
        M, w_old, w_new = combine_weights(m, mb)
        l_new = l * w_old + lb * w_new
        if normalised:
            # acc holds the normalised output so far: undo the old division,
            # add the block, divide by the new denominator (rows with no key stay 0)
            num = (l * w_old)[:, None] * acc + w_new[:, None] * pv
            acc = np.divide(num, l_new[:, None], out=np.zeros_like(num), where=l_new[:, None] > 0)
        else:
            acc = w_old[:, None] * acc + w_new[:, None] * pv
        m, l = np.atleast_1d(M), l_new
    return m, l, acc


def attention_deferred(q, k, v, query_widths=4, key_widths=3, scale=None, causal=False, key_len=None):
    """One head, query blocks independent of each other; within a block the key
    blocks are folded into unnormalised (m, l, acc), divided once at the end.
    Returns (O, LSE); rows without a visible key give O = 0, LSE = -inf."""
    N, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    vis = visibility(N, k.shape[0], causal, key_len)
    O = np.zeros((N, v.shape[1]))
    L = np.full(N, NEG_INF)
    for a, b in _blocks(N, query_widths):
        m, l, acc = _fold_keys(q[a:b], k, v, vis[a:b], scale, key_widths, normalised=False)
        seen = l > 0
        O[a:b][seen] = acc[seen] / l[seen, None]
        L[a:b][seen] = m[seen] + np.log(l[seen])
    return O, L


def attention_normalised(q, k, v, key_widths=3, scale=None, causal=False, key_len=None):
    """One head, key blocks outermost over all query rows, the output kept
    normalised after every block.  Returns (O, LSE)."""
    N, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    vis = visibility(N, k.shape[0], causal, key_len)
    m, l, O = _fold_keys(q, k, v, vis, scale, key_widths, normalised=True)
    L = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return O, L


# ------------------------------------------------------------------ fixtures
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
