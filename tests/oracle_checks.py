"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``check_*`` takes an oracle library handle and raises AssertionError on a
mismatch.  ``test_oracle.py`` runs them on the real oracle; the mutant test
runs them on copies of the oracle with a planted mistake and requires that at
least one check fails for every mutant.
"""
from __future__ import annotations

import math
import os

import numpy as np
import scipy.special
import torch

import oracle
import pagealgos as pa

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-12


def _golden(name):
    return pa.read_golden(os.path.join(GOLDEN, name))


def _floats(toks):
    return [float(t) for t in toks]


def _rng(seed):
    return np.random.default_rng(seed)


def _attn1(lib, q, k, v, **kw):
    """Single-head oracle call on fp64 [N,d] / [Nk,d] arrays."""
    O, L = oracle.attention(q[None, None], k[None, None], v[None, None], lib=lib, **kw)
    return O[0, 0], L[0, 0]


def _embed_scores(x):
    """Q, K, V so that the attention scores are x (scale 1) and O is softmax(x)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.size
    d = max(n, 1)
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((n, d)); k[:, 0] = x
    v = np.eye(n, d)
    return q, k, v


# --------------------------------------------------------------- worked examples
def check_worked_example(lib):
    g = _golden("softmax_worked_example.txt")
    dec = int(g["decimals"][0][0])
    tol = 0.5 * 10 ** (-dec) + 1e-12
    x = _floats(g["x"][0])
    y, m, l = oracle.softmax(x, lib=lib)
    assert m == float(g["max"][0][0])
    assert abs(l - float(g["sum"][0][0])) <= tol, l
    assert np.all(np.abs(y - _floats(g["y"][0])) <= tol), y
    assert np.all(np.abs(y * l - _floats(g["exponents"][0])) <= tol), y * l
    # the same numbers through the attention entry: O row = softmax, LSE = m + ln l
    q, k, v = _embed_scores(x)
    O, L = _attn1(lib, q, k, v, scale=1.0)
    assert np.all(np.abs(O[0, :3] - _floats(g["y"][0])) <= tol), O
    assert abs(math.exp(L[0] - m) - float(g["sum"][0][0])) <= tol, L
    assert abs(L[0] - (3.0 + math.log(math.exp(-2) + 1 + math.exp(-1)))) <= TIGHT


def check_four_element(lib):
    g = _golden("online_stats_example.txt")
    x = _floats(g["x"][0])
    y, m, l = oracle.softmax(x, lib=lib)
    assert m == float(g["m"][0][0])
    assert abs(l - float(g["l"][0][0])) <= float(g["page_atol"][0][0])
    # fp64 rounding of the printed value: the direct sum is ...109 in fp64
    assert abs(l - float(g["l"][0][0])) <= TIGHT
    assert np.allclose(np.exp(np.array(x) - m) / l, y, rtol=0, atol=TIGHT)
    assert np.allclose(y, scipy.special.softmax(x), rtol=0, atol=TIGHT)
    q, k, v = _embed_scores(x)
    _, L = _attn1(lib, q, k, v, scale=1.0)
    assert abs(L[0] - (5.0 + math.log(float(g["l"][0][0])))) <= TIGHT


def check_x153(lib):
    x = [1.0, 5.0, 3.0]
    y, m, l = oracle.softmax(x, lib=lib)
    l_closed = math.exp(-4.0) + 1.0 + math.exp(-2.0)
    assert m == 5.0 and abs(l - l_closed) <= TIGHT
    (mo, lo), _ = pa.scan(x)
    assert mo == m and abs(lo - l) <= TIGHT
    assert np.allclose(y, [math.exp(-4) / l_closed, 1 / l_closed, math.exp(-2) / l_closed],
                       rtol=0, atol=TIGHT)


# ------------------------------------------------------------------ chunk merge
def _chunk_matrix():
    g = _golden("merge_chunking.txt")
    rows, cols = int(g["rows"][0][0]), int(g["cols"][0][0])
    X = _rng(1805).standard_normal((rows, cols)) * float(g["sigma"][0][0])
    r1, npre = (int(t) for t in g["masked_prefix_row"][0])
    X[r1, :npre] = -np.inf
    X[int(g["fully_masked_row"][0][0]), :] = -np.inf
    return X, [int(t) for t in g["chunks"][0]], g


def check_chunk_merge(lib):
    X, widths, g = _chunk_matrix()
    assert sum(widths) == X.shape[1]
    full_row = int(g["fully_masked_row"][0][0])
    rng = _rng(37)
    parts = pa.segments(X, widths)                       # every row at once, per segment
    folded = pa.fold_left(parts)
    treed = pa.fold_tree(parts)
    for r in range(X.shape[0]):
        _, m, l = oracle.softmax(X[r], lib=lib)
        ref = scipy.special.logsumexp(X[r]) if np.isfinite(X[r]).any() else -np.inf
        row_parts = [(p[0][r], p[1][r]) for p in parts]
        candidates = [(folded[0][r], folded[1][r]), (treed[0][r], treed[1][r]), pa.scan(X[r])[0]]
        candidates += [pa.fold_random_tree(row_parts, rng) for _ in range(3)]
        for mc, lc in candidates:
            assert mc == m, (r, mc, m)
            assert abs(lc - l) <= TIGHT * max(1.0, l), (r, lc, l)
            assert not math.isnan(lc)
        assert abs(pa.lse((m, l)) - ref) <= TIGHT or (ref == -np.inf and pa.lse((m, l)) == -np.inf)
        if r == full_row:
            assert l == 0.0 and m == -math.inf
    # the same rows through the attention entry: a masked prefix is, up to key
    # order, a key length (softmax and LSE do not depend on key order)
    for r in range(X.shape[0]):
        fin = X[r][np.isfinite(X[r])]
        n = X.shape[1]
        xs = np.concatenate([fin, np.zeros(n - fin.size)])
        q, k, v = _embed_scores(xs)
        O, L = oracle.attention(q[None, None], k[None, None], v[None, None], scale=1.0,
                                key_lens=[fin.size], lib=lib)
        ref = scipy.special.logsumexp(fin) if fin.size else -np.inf
        if fin.size:
            assert abs(L[0, 0, 0] - ref) <= TIGHT
            assert np.allclose(O[0, 0, 0, :fin.size], scipy.special.softmax(fin), rtol=0, atol=TIGHT)
        else:
            assert L[0, 0, 0] == -np.inf and np.all(O == 0) and not np.isnan(O).any()


def check_merge_guard_negative_control(lib):
    # without the guard the fully masked side gives NaN; with it, (m, l) = (-inf, 0)
    _, m, l = oracle.softmax([-np.inf] * 5, lib=lib)
    assert m == -np.inf and l == 0.0
    _, nl = pa.combine_unguarded((m, l), (m, l))
    assert math.isnan(nl)
    gm, gl = pa.combine((m, l), (m, l))
    assert gm == -np.inf and gl == 0.0


# ----------------------------------------------------------------- tiled shapes
def check_tiled_shapes(lib):
    g = _golden("tiled_v1_shapes.txt")
    Br, Bc = int(g["Br"][0][0]), int(g["Bc"][0][0])
    for idx, sh in enumerate(g["shape"]):
        N, Nk, d = (int(t) for t in sh)
        r = _rng(100 + idx)
        q, k, v = r.standard_normal((N, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
        for causal in (False, True):
            for kl in (None, max(Nk - 2, 0), 1):
                O, L = _attn1(lib, q, k, v, causal=causal, key_lens=None if kl is None else [kl])
                O1, L1 = pa.attention_normalised(q, k, v, Bc, causal=causal, key_len=kl)
                O2, L2 = pa.attention_deferred(q, k, v, Br, Bc, causal=causal, key_len=kl)
                # ragged block widths, cycled, for both orders
                O3, L3 = pa.attention_normalised(q, k, v, [2, 1, 4], causal=causal, key_len=kl)
                O4, L4 = pa.attention_deferred(q, k, v, [3, 1], [1, 5, 2], causal=causal, key_len=kl)
                for Ot, Lt in ((O1, L1), (O2, L2), (O3, L3), (O4, L4)):
                    assert np.allclose(O, Ot, rtol=0, atol=TIGHT), (N, Nk, d, causal, kl)
                    fin = np.isfinite(L)
                    assert np.array_equal(fin, np.isfinite(Lt))
                    assert np.allclose(L[fin], Lt[fin], rtol=0, atol=TIGHT)
        # the library attention (fp64, no mask), as on the page
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0]
        O, L = _attn1(lib, q, k, v)
        assert np.allclose(O, ref.numpy(), rtol=0, atol=float(g["page_atol"][0][0]))
        assert np.allclose(O, ref.numpy(), rtol=0, atol=TIGHT)
        lse_ref = scipy.special.logsumexp(q @ k.T / math.sqrt(d), axis=1)
        assert np.allclose(L, lse_ref, rtol=0, atol=TIGHT)


# ----------------------------------------------------------------- closed forms
def check_closed_forms(lib):
    r = _rng(7)
    d = 6
    # one key: O = v0, LSE = s0
    q, k, v = r.standard_normal((5, d)), r.standard_normal((1, d)), r.standard_normal((1, d))
    O, L = _attn1(lib, q, k, v, scale=0.7)
    assert np.allclose(O, np.repeat(v, 5, 0), rtol=0, atol=TIGHT)
    assert np.allclose(L, 0.7 * (q @ k[0]), rtol=0, atol=TIGHT)
    # key length 1: O = v0 whatever Nk
    q, k, v = r.standard_normal((4, d)), r.standard_normal((9, d)), r.standard_normal((9, d))
    O, L = _attn1(lib, q, k, v, key_lens=[1])
    assert np.allclose(O, np.repeat(v[:1], 4, 0), rtol=0, atol=TIGHT)
    # causal, N == Nk: row 0 sees key 0 only; row 1 sees keys 0 and 1
    q, k, v = r.standard_normal((7, d)), r.standard_normal((7, d)), r.standard_normal((7, d))
    sc = 1 / math.sqrt(d)
    O, L = _attn1(lib, q, k, v, causal=True)
    assert np.allclose(O[0], v[0], rtol=0, atol=TIGHT)
    assert abs(L[0] - sc * q[0] @ k[0]) <= TIGHT
    s = sc * (k[:2] @ q[1])
    w = np.exp(s - s.max()); w /= w.sum()
    assert np.allclose(O[1], w @ v[:2], rtol=0, atol=TIGHT)
    # causal with N > Nk: queries are the last N positions, so the first N - Nk rows see nothing
    q, k, v = r.standard_normal((6, d)), r.standard_normal((4, d)), r.standard_normal((4, d))
    O, L = _attn1(lib, q, k, v, causal=True)
    assert np.all(O[:2] == 0) and np.all(L[:2] == -np.inf)
    assert np.allclose(O[2], v[0], rtol=0, atol=TIGHT)
    # causal with N < Nk: the last query sees every key
    q, k, v = r.standard_normal((3, d)), r.standard_normal((8, d)), r.standard_normal((8, d))
    O, L = _attn1(lib, q, k, v, causal=True)
    O_full, L_full = _attn1(lib, q[2:], k, v)
    assert np.allclose(O[2], O_full[0], rtol=0, atol=TIGHT) and abs(L[2] - L_full[0]) <= TIGHT
    O6, _ = _attn1(lib, q[:1], k[:6], v[:6])
    assert np.allclose(O[0], O6[0], rtol=0, atol=TIGHT)
    # zero query: uniform weights over the visible keys
    q, k, v = np.zeros((3, d)), r.standard_normal((10, d)), r.standard_normal((10, d))
    O, L = _attn1(lib, q, k, v, key_lens=[7])
    assert np.allclose(O, np.repeat(v[:7].mean(0, keepdims=True), 3, 0), rtol=0, atol=TIGHT)
    assert np.allclose(L, math.log(7), rtol=0, atol=TIGHT)
    # identical keys: uniform weights, LSE = s + ln Nk
    q, k1, v = r.standard_normal((2, d)), r.standard_normal((1, d)), r.standard_normal((5, d))
    k = np.repeat(k1, 5, 0)
    O, L = _attn1(lib, q, k, v)
    assert np.allclose(O, np.repeat(v.mean(0, keepdims=True), 2, 0), rtol=0, atol=TIGHT)
    assert np.allclose(L, sc * (q @ k1[0]) + math.log(5), rtol=0, atol=TIGHT)
    # identity values (d >= Nk): the output row is the probability row
    q, k = r.standard_normal((4, 8)), r.standard_normal((5, 8))
    v = np.eye(5, 8)
    O, L = _attn1(lib, q, k, v, scale=0.3)
    P = scipy.special.softmax(0.3 * q @ k.T, axis=1)
    assert np.allclose(O[:, :5], P, rtol=0, atol=TIGHT) and np.all(O[:, 5:] == 0)
    # no keys at all: every row fully masked
    O, L = oracle.attention(np.ones((1, 2, 3, 4)), np.ones((1, 2, 0, 4)), np.ones((1, 2, 0, 4)), lib=lib)
    assert np.all(O == 0) and np.all(L == -np.inf)
    # key length 0 on one batch only
    q, k, v = r.standard_normal((2, 1, 3, d)), r.standard_normal((2, 1, 4, d)), r.standard_normal((2, 1, 4, d))
    O, L = oracle.attention(q, k, v, key_lens=[4, 0], lib=lib)
    assert np.all(O[1] == 0) and np.all(L[1] == -np.inf) and np.all(np.isfinite(L[0]))


# ------------------------------------------------------------------- invariants
def check_invariants(lib):
    r = _rng(11)
    N, Nk, d = 5, 9, 7
    q, k, v = r.standard_normal((N, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    O, L = _attn1(lib, q, k, v)
    perm = r.permutation(Nk)
    Op, Lp = _attn1(lib, q, k[perm], v[perm])
    assert np.allclose(O, Op, rtol=0, atol=TIGHT) and np.allclose(L, Lp, rtol=0, atol=TIGHT)
    # convex combination of the value rows
    assert np.all(O <= v.max(0) + TIGHT) and np.all(O >= v.min(0) - TIGHT)
    # LSE >= max score, LSE <= max score + ln Nk
    s = q @ k.T / math.sqrt(d)
    assert np.all(L >= s.max(1) - TIGHT) and np.all(L <= s.max(1) + math.log(Nk) + TIGHT)
    # every key twice: same output, LSE + ln 2
    O2, L2 = _attn1(lib, q, np.concatenate([k, k]), np.concatenate([v, v]))
    assert np.allclose(O, O2, rtol=0, atol=TIGHT) and np.allclose(L + math.log(2), L2, rtol=0, atol=TIGHT)
    # adding a constant vector to V adds it to O (weights sum to 1)
    c = r.standard_normal(d)
    O3, _ = _attn1(lib, q, k, v + c)
    assert np.allclose(O3, O + c, rtol=0, atol=1e-11)


def check_torch_sdpa(lib):
    r = _rng(23)
    B, H, N, Nk, d = 2, 3, 7, 11, 5
    q, k, v = (r.standard_normal(s) for s in ((B, H, N, d), (B, H, Nk, d), (B, H, Nk, d)))
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    O, L = oracle.attention(q, k, v, lib=lib)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    assert np.allclose(O, ref.numpy(), rtol=0, atol=TIGHT)
    lse = torch.logsumexp(torch.matmul(tq, tk.transpose(-1, -2).contiguous()) / math.sqrt(d), dim=-1)
    assert np.allclose(L, lse.numpy(), rtol=0, atol=TIGHT)
    # causal, N == Nk (the library aligns the mask at the top-left; equal here)
    q2, k2, v2 = q[:, :, :6], k[:, :, :6], v[:, :, :6]
    O, L = oracle.attention(q2, k2, v2, causal=True, lib=lib)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q2), torch.from_numpy(k2), torch.from_numpy(v2), is_causal=True)
    assert np.allclose(O, ref.numpy(), rtol=0, atol=TIGHT)
    # causal, N < Nk: bottom-right alignment as an explicit boolean mask
    mask = np.arange(Nk)[None, :] <= np.arange(N)[:, None] + (Nk - N)
    O, L = oracle.attention(q, k, v, causal=True, lib=lib)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask))
    assert np.allclose(O, ref.numpy(), rtol=0, atol=TIGHT)


def check_bf16_widening(lib):
    g = torch.Generator().manual_seed(5)
    q = (torch.randn(1, 2, 5, 8, generator=g) * 3).to(torch.bfloat16)
    k = torch.randn(1, 2, 6, 8, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 2, 6, 8, generator=g).to(torch.bfloat16)
    Ob, Lb = oracle.attention(q, k, v, causal=True, lib=lib)
    Od, Ld = oracle.attention(q.double(), k.double(), v.double(), causal=True, lib=lib)
    assert np.array_equal(Ob, Od) and np.array_equal(Lb, Ld)
    Of, Lf = oracle.attention(q.float(), k.float(), v.float(), causal=True, lib=lib)
    assert np.array_equal(Of, Od) and np.array_equal(Lf, Ld)


def check_rows_and_threads(lib):
    r = _rng(31)
    B, H, N, Nk, d = 2, 2, 9, 13, 4
    q, k, v = (r.standard_normal(s) for s in ((B, H, N, d), (B, H, Nk, d), (B, H, Nk, d)))
    O, L = oracle.attention(q, k, v, causal=True, key_lens=[10, 3], nthreads=1, lib=lib)
    O8, L8 = oracle.attention(q, k, v, causal=True, key_lens=[10, 3], nthreads=8, lib=lib)
    assert np.array_equal(O, O8) and np.array_equal(L, L8)
    rows = [0, 5, 17, 20, 35, 2 * 2 * 9 - 1]
    Or, Lr = oracle.attention(q, k, v, causal=True, key_lens=[10, 3], rows=rows, lib=lib)
    assert np.array_equal(Or, O.reshape(-1, d)[rows]) and np.array_equal(Lr, L.reshape(-1)[rows])
    # key length k equals truncating K and V to their first k rows
    for b, kl in enumerate([10, 3]):
        Ot, Lt = oracle.attention(q[b:b + 1], k[b:b + 1, :, :kl], v[b:b + 1, :, :kl], lib=lib)
        Ok, Lk = oracle.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], key_lens=[kl], lib=lib)
        assert np.array_equal(Ot, Ok) and np.array_equal(Lt, Lk)
    # per-batch key lengths index the batch, not the head
    Ob, Lb = oracle.attention(q, k, v, key_lens=[13, 2], lib=lib)
    O0, L0 = oracle.attention(q[:1], k[:1], v[:1], lib=lib)
    O1, L1 = oracle.attention(q[1:], k[1:, :, :2], v[1:, :, :2], lib=lib)
    assert np.array_equal(Ob[0], O0[0]) and np.array_equal(Ob[1], O1[0])


def check_softmax_rows(lib):
    # every row equals the single-vector softmax; LSE is the library logsumexp
    X, widths, g = _chunk_matrix()
    Y, L = oracle.softmax_rows(X, lib=lib)
    for r in range(X.shape[0]):
        y, m, l = oracle.softmax(X[r], lib=lib)
        assert np.array_equal(Y[r], y)
        ref = scipy.special.logsumexp(X[r]) if np.isfinite(X[r]).any() else -np.inf
        assert (L[r] == -np.inf and ref == -np.inf) or abs(L[r] - ref) <= TIGHT
    fin = np.isfinite(X).any(axis=1)
    assert np.allclose(Y[fin], scipy.special.softmax(np.where(np.isfinite(X), X, -np.inf)[fin], axis=1),
                       rtol=0, atol=TIGHT)
    # worked example through the rows entry, fp32 and bf16 storage widen exactly
    Yw, Lw = oracle.softmax_rows(np.array([[1.0, 3.0, 2.0], [1.0, 3.0, 2.0]], dtype=np.float32), lib=lib)
    gw = _golden("softmax_worked_example.txt")
    tol = 0.5 * 10 ** (-int(gw["decimals"][0][0])) + 1e-12
    assert np.all(np.abs(Yw - _floats(gw["y"][0])) <= tol)
    assert abs(math.exp(Lw[0] - 3.0) - float(gw["sum"][0][0])) <= tol
    xb = torch.tensor([[0.5, -2.0, 7.25, 3.0]]).to(torch.bfloat16)
    Yb, Lb = oracle.softmax_rows(xb, lib=lib)
    assert abs(Lb[0] - scipy.special.logsumexp(xb.double().numpy()[0])) <= TIGHT
    # shift invariance: softmax(x + c) = softmax(x), LSE(x + c) = LSE(x) + c
    r = _rng(41).standard_normal((3, 50))
    Y1, L1 = oracle.softmax_rows(r, lib=lib)
    Y2, L2 = oracle.softmax_rows(r + 7.5, lib=lib)
    assert np.allclose(Y1, Y2, rtol=0, atol=TIGHT) and np.allclose(L1 + 7.5, L2, rtol=0, atol=1e-11)
    # empty rows
    Ye, Le = oracle.softmax_rows(np.zeros((2, 0)), lib=lib)
    assert Ye.shape == (2, 0) and np.all(Le == -np.inf)


# --------------------------------------------------------------------- backward
def _bwd_case(r, B, H, N, Nk, d):
    return (r.standard_normal((B, H, N, d)), r.standard_normal((B, H, Nk, d)),
            r.standard_normal((B, H, Nk, d)), r.standard_normal((B, H, N, d)))


def _loss(lib, q, k, v, do, **kw):
    O, _ = oracle.attention(q, k, v, lib=lib, nthreads=1, **kw)
    return float((O * do).sum())


BWD_CASES = [
    dict(B=1, H=2, N=5, Nk=4, d=3, causal=False, key_lens=None, scale=None),
    dict(B=2, H=1, N=4, Nk=6, d=3, causal=True, key_lens=None, scale=0.7),
    dict(B=2, H=1, N=6, Nk=4, d=2, causal=True, key_lens=None, scale=None),   # N > Nk: rows 0, 1 see nothing
    dict(B=2, H=1, N=4, Nk=5, d=3, causal=False, key_lens=[3, 0], scale=None),
    dict(B=1, H=1, N=5, Nk=5, d=4, causal=True, key_lens=[4], scale=1.3),
]


def check_backward_finite_differences(lib):
    # central differences of the (separately pinned) forward: L = sum dO . O
    r = _rng(77)
    h = 1e-5
    for cs in BWD_CASES:
        B, H, N, Nk, d = cs["B"], cs["H"], cs["N"], cs["Nk"], cs["d"]
        kw = dict(scale=cs["scale"], causal=cs["causal"], key_lens=cs["key_lens"])
        q, k, v, do = _bwd_case(r, B, H, N, Nk, d)
        dQ, dK, dV = oracle.attention_backward(q, k, v, do, lib=lib, nthreads=1, **kw)
        for which, g in ((0, dQ), (1, dK), (2, dV)):
            base = [q, k, v]
            x = base[which]
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                argp, argm = list(base), list(base)
                argp[which], argm[which] = xp, xm
                fd = (_loss(lib, *argp, do, **kw) - _loss(lib, *argm, do, **kw)) / (2 * h)
                assert abs(fd - g[idx]) <= 1e-6 * (1.0 + abs(g[idx])), (cs, which, idx, fd, g[idx])


def check_backward_torch_autograd(lib):
    # the library's automatic differentiation of the same masked attention, fp64
    r = _rng(78)
    for cs in BWD_CASES:
        B, H, N, Nk, d = cs["B"], cs["H"], cs["N"], cs["Nk"], cs["d"]
        scale = cs["scale"] if cs["scale"] is not None else 1.0 / math.sqrt(d)
        q, k, v, do = _bwd_case(r, B, H, N, Nk, d)
        dQ, dK, dV = oracle.attention_backward(q, k, v, do, scale=scale, causal=cs["causal"],
                                               key_lens=cs["key_lens"], lib=lib)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
        vis = torch.ones(B, 1, N, Nk, dtype=torch.bool)
        if cs["causal"]:
            i = torch.arange(N)[:, None]
            j = torch.arange(Nk)[None, :]
            vis = vis & (j <= i + (Nk - N))
        if cs["key_lens"] is not None:
            kl = torch.tensor(cs["key_lens"])[:, None, None, None]
            vis = vis & (torch.arange(Nk)[None, None, None, :] < kl)
        s = s.masked_fill(~vis, float("-inf"))
        any_vis = vis.any(dim=-1, keepdim=True)
        p = torch.where(any_vis, torch.softmax(torch.where(any_vis, s, torch.zeros_like(s)), dim=-1),
                        torch.zeros_like(s))
        o = torch.matmul(p, tv)
        (o * torch.from_numpy(do)).sum().backward()
        for g, t in ((dQ, tq), (dK, tk), (dV, tv)):
            assert np.allclose(g, t.grad.numpy(), rtol=0, atol=1e-12), cs


def check_backward_closed_forms(lib):
    r = _rng(79)
    # one key: softmax is constant 1, so no gradient reaches Q or K; dV = sum of dO
    q, k, v, do = _bwd_case(r, 1, 2, 6, 1, 4)
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, lib=lib)
    assert np.abs(dQ).max() <= 1e-14 and np.abs(dK).max() <= 1e-14
    assert np.allclose(dV[:, :, 0], do.sum(axis=2), rtol=0, atol=1e-13)
    # identical value rows: O = v whatever P is, so dS = 0
    q, k, v, do = _bwd_case(r, 1, 1, 5, 7, 3)
    v[:] = v[:, :, :1, :]
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, lib=lib)
    assert np.abs(dQ).max() <= 1e-13 and np.abs(dK).max() <= 1e-13
    # zero upstream gradient
    dQ, dK, dV = oracle.attention_backward(q, k, v, np.zeros_like(do), lib=lib)
    assert not dQ.any() and not dK.any() and not dV.any()
    # invariants: key shift leaves every softmax unchanged, so sum_j dK_j = 0;
    # a value shift moves every visible row's output, so sum_j dV_j = sum_i dO_i
    for cs in BWD_CASES:
        q, k, v, do = _bwd_case(r, cs["B"], cs["H"], cs["N"], cs["Nk"], cs["d"])
        kw = dict(scale=cs["scale"], causal=cs["causal"], key_lens=cs["key_lens"])
        dQ, dK, dV = oracle.attention_backward(q, k, v, do, lib=lib, **kw)
        _, L = oracle.attention(q, k, v, lib=lib, **kw)
        seen = np.isfinite(L)[..., None]
        assert np.abs(dK.sum(axis=2)).max() <= 1e-12, cs
        assert np.allclose(dV.sum(axis=2), (do * seen).sum(axis=2), rtol=0, atol=1e-12), cs
        assert np.all(dQ[~np.isfinite(L)] == 0.0), cs
    # Nk = 0: nothing is visible
    q, k, v, do = _bwd_case(r, 1, 1, 3, 0, 2)
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, lib=lib)
    assert not dQ.any() and dK.shape == (1, 1, 0, 2)


def check_backward_heads_and_widening(lib):
    r = _rng(80)
    q, k, v, do = _bwd_case(r, 2, 3, 7, 9, 4)
    full = oracle.attention_backward(q, k, v, do, causal=True, key_lens=[9, 4], lib=lib)
    sub = oracle.attention_backward(q, k, v, do, causal=True, key_lens=[9, 4], heads=[4, 0], lib=lib)
    for f, s_ in zip(full, sub):
        fl = f.reshape(6, *f.shape[2:])
        assert np.array_equal(s_[0], fl[4]) and np.array_equal(s_[1], fl[0])
    # bf16 and fp32 storage widen exactly: same result as the widened fp64 values
    tb = [torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v, do)]
    gb = oracle.attention_backward(*tb, scale=0.5, lib=lib)
    g64 = oracle.attention_backward(*[t.double().numpy() for t in tb], scale=0.5, lib=lib)
    assert all(np.array_equal(a, b) for a, b in zip(gb, g64))
    tf = [x.astype(np.float32) for x in (q, k, v, do)]
    gf = oracle.attention_backward(*tf, scale=0.5, lib=lib)
    g64 = oracle.attention_backward(*[x.astype(np.float64) for x in tf], scale=0.5, lib=lib)
    assert all(np.array_equal(a, b) for a, b in zip(gf, g64))


ALL_CHECKS = [
    check_worked_example, check_four_element, check_x153, check_chunk_merge,
    check_merge_guard_negative_control, check_tiled_shapes, check_closed_forms,
    check_invariants, check_torch_sdpa, check_bf16_widening, check_rows_and_threads,
    check_softmax_rows, check_backward_finite_differences, check_backward_torch_autograd,
    check_backward_closed_forms, check_backward_heads_and_widening,
]
