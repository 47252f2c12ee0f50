"""Helpers for the GPU parity tests: run the HIP path, run the oracle on the
same bytes, compare to the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import attention_forward_online_amd as fa
import oracle

# Tolerances on max |GPU - oracle| (fp64 oracle on the same stored inputs):
#   fp32 path: 1e-5 on O and on LSE;
#   bf16 path (bf16 operands, fp32 accumulation, bf16 O): 2e-2 on O, 1e-3 on LSE.
TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (2e-2, 1e-3)}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_host(t: torch.Tensor) -> torch.Tensor:
    return t.detach().to("cpu")


def compare(o_gpu, lse_gpu, O_ref, L_ref, dtype, what=""):
    """Element-wise check of GPU outputs (any shape, rows last-but-one) against
    the oracle; returns (max |dO|, max |dLSE|) over rows with visible keys."""
    tol_o, tol_l = TOL[dtype]
    o = to_host(o_gpu).double().numpy().reshape(O_ref.shape)
    l = to_host(lse_gpu).double().numpy().reshape(L_ref.shape)
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(l).any(), f"{what}: NaN in LSE"
    masked = np.isneginf(L_ref)
    # fully masked rows: exactly O = 0 and LSE = -inf
    assert np.array_equal(np.isneginf(l), masked), f"{what}: -inf pattern of LSE differs"
    if masked.any():
        assert np.all(o[masked] == 0.0), f"{what}: masked rows not exactly zero"
    vis = ~masked
    eo = float(np.abs(o[vis] - O_ref[vis]).max()) if vis.any() else 0.0
    el = float(np.abs(l[vis] - L_ref[vis]).max()) if vis.any() else 0.0
    assert eo <= tol_o, f"{what}: max |dO| = {eo:.3e} > {tol_o:g}"
    assert el <= tol_l, f"{what}: max |dLSE| = {el:.3e} > {tol_l:g}"
    return eo, el


def forward_and_check(inp, causal, scale=None, what="", rows=None):
    q, k, v, kl = inp["q"], inp["k"], inp["v"], inp["key_lens"]
    B, H, N, d = q.shape
    say(f"[gpu] fa_forward {what} B={B} H={H} N={N} Nk={k.shape[2]} d={d} {q.dtype} "
        f"causal={causal} key_lens={None if kl is None else kl.tolist()}")
    o, lse = fa.attention(q, k, v, scale=scale, causal=causal, key_lens=kl)
    torch.cuda.synchronize()
    qh, kh, vh = to_host(q), to_host(k), to_host(v)
    klh = None if kl is None else to_host(kl).tolist()
    sc = scale if scale is not None else float(np.float32(1.0 / np.sqrt(d)))
    if rows is None:
        O_ref, L_ref = oracle.attention(qh, kh, vh, scale=sc, causal=causal, key_lens=klh)
        return compare(o, lse, O_ref, L_ref, q.dtype, what) + (o, lse)
    O_ref, L_ref = oracle.attention(qh, kh, vh, scale=sc, causal=causal, key_lens=klh, rows=rows)
    o_rows = to_host(o).reshape(-1, d)[torch.as_tensor(rows)]
    l_rows = to_host(lse).reshape(-1)[torch.as_tensor(rows)]
    return compare(o_rows, l_rows, O_ref, L_ref, q.dtype, what) + (o, lse)


def sample_rows(B, H, N, per_head=6, seed=0, bh_limit=None):
    """Flat row indices: tile edges, first/last rows and random rows of a set of heads."""
    rng = np.random.default_rng(seed)
    heads = range(B * H) if bh_limit is None else rng.choice(B * H, size=min(bh_limit, B * H), replace=False)
    rows = []
    for bh in heads:
        cand = {0, N - 1, min(127, N - 1), min(128, N - 1), N // 2}
        cand |= set(rng.integers(0, N, size=per_head).tolist())
        rows += [int(bh) * N + i for i in sorted(cand)]
    return rows
