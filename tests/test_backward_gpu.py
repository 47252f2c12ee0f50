"""GPU parity of the bf16 attention backward (fa_backward, d = 64 and 128) against the
fp64 oracle's exact gradients on the same stored inputs.

The GPU path starts from its own forward (bf16 O, fp32 LSE), rounds P and dS to
bf16 as MFMA operands and accumulates in fp32 (at d = 128 the dK/dV kernel forms
dS from P rounded to fp16, 2^-12, not 2^-9); dQ, dK, dV are stored in bf16.
Tolerance per gradient tensor G (bf16): max |G - G_ref| <= 8e-3 * max |G_ref| + 1e-3.
Derivation: the stored gradient is rounded to bf16 (up to 2^-9 = 0.2% of
max |G|), and every product in its sum carries one bf16 rounding of P or dS
(relative 2^-9, of mixed sign over up to a few thousand terms); measured at
most 0.68% of max |G_ref| over every case here (a d = 64 dQ entry near 1, at
0.77 of the bound).  fp32 path (fp32 throughout, from the fp32 forward's
O and LSE): max |G - G_ref| <= 2e-5 * max |G_ref| + 1e-6 (fp32 sums over up to
a few thousand terms; the forward's LSE and O errors of ~1e-6 enter P and D;
measured at most 1.2e-6 of max |G_ref|).
Rows and keys that see nothing must be exactly 0.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import attention_forward_online_amd as fa
import oracle
from attention_forward_online_amd import synth
from gpu_common import say, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOLS = {torch.bfloat16: (8e-3, 1e-3), torch.float32: (2e-5, 1e-6)}


def make(B, H, N, Nk, seed, key_lens=None, d=64, dtype=torch.bfloat16):
    inp = synth.random_case(B, H, N, Nk, d, dtype, seed=seed, device=DEV, key_lens=key_lens)
    do = synth.randn_slices((B, H, N, d), 1.0, dtype, seed, f"bwd_{B}_{H}_{N}_{Nk}_{d}", "do", DEV)
    return inp["q"], inp["k"], inp["v"], do, inp["key_lens"]


def host_threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, 32))


def run_and_check(q, k, v, do, kl, causal, scale=None, heads=None, what="", nthreads=None):
    B, H, N, d = q.shape
    Nk = k.shape[2]
    say(f"[gpu] fa_backward {what} B={B} H={H} N={N} Nk={Nk} causal={causal} "
        f"key_lens={None if kl is None else kl.tolist()} scale={scale}")
    o, lse = fa.attention(q, k, v, scale=scale, causal=causal, key_lens=kl)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, scale=scale, causal=causal, key_lens=kl)
    torch.cuda.synchronize()
    sc = scale if scale is not None else float(np.float32(1.0 / np.sqrt(d)))
    REL, ABS = TOLS[q.dtype]
    klh = None if kl is None else to_host(kl).tolist()
    ref = oracle.attention_backward(to_host(q), to_host(k), to_host(v), to_host(do), scale=sc,
                                    causal=causal, key_lens=klh, heads=heads, nthreads=nthreads)
    got = [to_host(t).double().numpy() for t in (dq, dk, dv)]
    if heads is not None:
        got = [g.reshape(B * H, *g.shape[2:])[heads] for g in got]
        ref = [r.reshape(len(heads), *r.shape[1:]) for r in ref]
    # rows that see no key and keys that no query sees get exactly 0
    klv = np.array(klh if klh is not None else [Nk] * B)
    off = Nk - N
    row_dead = np.zeros((B, H, N), dtype=bool)
    key_dead = np.zeros((B, H, Nk), dtype=bool)
    for bb in range(B):
        kl_b = int(min(max(klv[bb], 0), Nk))
        i = np.arange(N)
        nvis = np.minimum(kl_b, i + off + 1) if causal else np.full(N, kl_b)
        row_dead[bb] = (nvis <= 0)[None, :]
        j = np.arange(Nk)
        seen = (j < kl_b) & ((j <= N - 1 + off) if causal else True) & (N > 0)
        key_dead[bb] = (~seen)[None, :]
    if heads is not None:
        row_dead = row_dead.reshape(B * H, N)[heads]
        key_dead = key_dead.reshape(B * H, Nk)[heads]
    errs = []
    for name, g, r, dead in zip(("dQ", "dK", "dV"), got, ref, (row_dead, key_dead, key_dead)):
        g = g.reshape(r.shape)
        assert not np.isnan(g).any(), f"{what}: NaN in {name}"
        e = float(np.abs(g - r).max()) if r.size else 0.0
        scale_r = float(np.abs(r).max()) if r.size else 0.0
        errs.append((name, e, scale_r))
        assert e <= REL * scale_r + ABS, f"{what}: {name} max err {e:.3e} vs max |ref| {scale_r:.3e}"
        dead = dead.reshape(r.shape[:-1])
        assert np.all(r[dead] == 0.0)
        assert np.all(g[dead] == 0.0), f"{what}: {name} rows without any gradient not exactly 0"
    say(f"    " + "  ".join(f"{n}: max|err| {e:.2e} / max|ref| {s:.2e}" for n, e, s in errs))
    return errs


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,Nk", [(128, 128), (200, 200), (77, 130), (130, 77), (256, 320), (64, 1)])
def test_shapes(N, Nk, causal):
    q, k, v, do, kl = make(1, 2, N, Nk, seed=N * 1000 + Nk)
    run_and_check(q, k, v, do, kl, causal, what=f"shapes {N}x{Nk}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,Nk", [(128, 128), (77, 130), (130, 77), (300, 300)])
def test_shapes_d128(N, Nk, causal):
    q, k, v, do, kl = make(1, 2, N, Nk, seed=N * 1000 + Nk + 1, d=128)
    run_and_check(q, k, v, do, kl, causal, what=f"d128 shapes {N}x{Nk}")


@pytest.mark.parametrize("causal", [False, True])
def test_key_lens_d128(causal):
    q, k, v, do, kl = make(2, 2, 150, 190, seed=17, key_lens=[101, 0], d=128)
    run_and_check(q, k, v, do, kl, causal, what="d128 key_lens")


@pytest.mark.parametrize("causal", [False, True])
def test_key_lens_and_empty_batch(causal):
    q, k, v, do, kl = make(2, 2, 150, 190, seed=7, key_lens=[101, 0])
    run_and_check(q, k, v, do, kl, causal, what="key_lens")


def test_scale_and_ragged_batch_heads():
    q, k, v, do, kl = make(3, 3, 96, 160, seed=11)
    run_and_check(q, k, v, do, kl, False, scale=0.05, what="scale 0.05")
    run_and_check(q, k, v, do, kl, True, scale=0.3, what="scale 0.3 causal")


@pytest.mark.parametrize("d", [64, 128])
def test_empty_sides(d):
    # no queries: dK = dV = 0; no keys: dQ = 0
    q, k, v, do, kl = make(1, 2, 0, 70, seed=3, d=d)
    o, lse = fa.attention(q, k, v)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert dq.shape == q.shape and torch.all(dk == 0) and torch.all(dv == 0)
    q, k, v, do, kl = make(1, 2, 50, 0, seed=4, d=d)
    o, lse = fa.attention(q, k, v)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.shape == k.shape


@pytest.mark.parametrize("d", [64, 128])
def test_deterministic(d):
    # no atomics anywhere: two calls give the same bits (at d = 128 with P handed
    # between the two waves of each key group through LDS)
    q, k, v, do, kl = make(2, 4, 300, 300, seed=5, d=d)
    o, lse = fa.attention(q, k, v, causal=True)
    a = fa.attention_backward(q, k, v, o, lse, do, causal=True)
    b = fa.attention_backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("extra_heads", [0, 1])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_split_grid_boundary(d, causal, extra_heads):
    # a grid of at most one block per CU runs each block's tiles in two halves whose
    # partial sums are added at the end: the key tiles of a 128-query dQ block, and
    # at d = 64 the query tiles of a 128-key dK/dV block (N = 300 and Nk = 330 give
    # three blocks per head in both kernels; the d = 128 dK/dV kernel runs its
    # 8-wave workgroups at any grid size); one more head per batch puts the same
    # inputs on the unsplit path.  Key lengths: one tile (split 1 / 0), two tiles, an odd count, all;
    # causal with Nk > N puts the diagonal in the second half.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, N, Nk = 4, 300, 330
    H = cus // (B * 3) + extra_heads
    q, k, v, do, kl = make(B, H, N, Nk, seed=61 + d, key_lens=[1, 65, 200, 330], d=d)
    heads = sorted({0, 1, H - 1, H + 2, 2 * H + 5, 3 * H + H // 2, B * H - 1})
    run_and_check(q, k, v, do, kl, causal, heads=heads,
                  what=f"{B * H * 3} blocks vs {cus} CUs")


@pytest.mark.parametrize("B,H,N,Nk,d", [(64, 2, 70, 150, 64), (3, 5, 257, 300, 128),
                                          (200, 2, 70, 150, 64)])
def test_key_length_launch_order(B, H, N, Nk, d):
    # non-causal grids with key lengths go out batch by batch in descending order of
    # visible keys in both backward kernels (each workgroup ranks the batches itself):
    # every (head, block) once, with tied, empty, past-Nk and negative key lengths
    rng = np.random.default_rng(B * 1000 + N)
    kl = [int(x) for x in rng.choice([0, 1, 37, Nk // 2, Nk // 2, Nk, Nk + 9, -3], size=B)]
    q, k, v, do, klt = make(B, H, N, Nk, seed=B + d, key_lens=kl, d=d)
    run_and_check(q, k, v, do, klt, False, what=f"key-length order B={B}")


@pytest.mark.parametrize("B,H,N,Nk,d,causal", [(1, 16, 1000, 4500, 128, True), (1, 16, 9000, 300, 64, False)])
def test_grouped_head_order(B, H, N, Nk, d, causal):
    # heads whose streamed K/V (dQ kernel) or Q/dO (dK/dV kernel) exceed an XCD's
    # L2 go in groups of one head: every (head, block) once; three heads in full
    q, k, v, do, kl = make(B, H, N, Nk, seed=N + Nk, d=d)
    run_and_check(q, k, v, do, kl, causal, heads=[0, 7, 15], what=f"grouped order N={N} Nk={Nk}")


def test_full_size_d64_causal_shape():
    # B4 H16 N=Nk=2048 d64 causal, the bench's backward workload: every element
    # of dQ, dK and dV (the oracle takes a few seconds on the host's cores)
    w = synth.WORKLOADS["causal_bf16_b4h16_n2048_d64"]
    inp = synth.make_inputs(w, device=DEV)
    do = synth.randn_slices((w.B, w.H, w.N, w.d), 1.0, torch.bfloat16, 0, w.name, "do", DEV)
    run_and_check(inp["q"], inp["k"], inp["v"], do, None, True, what="d64 causal shape, every head",
                  nthreads=host_threads())


def test_full_size_long_d128_shape():
    # B1 H32 N=Nk=8192 d128 causal (the headline prefill's shape), the bench's
    # second backward workload: every element of dQ, dK and dV (about a minute
    # of fp64 oracle work on 16 cores)
    w = synth.WORKLOADS["causal_bf16_b1h32_n8192_d128"]
    inp = synth.make_inputs(w, device=DEV)
    do = synth.randn_slices((w.B, w.H, w.N, w.d), 1.0, torch.bfloat16, 0, w.name, "do", DEV)
    run_and_check(inp["q"], inp["k"], inp["v"], do, None, True, what="8192-long d128, every head",
                  nthreads=host_threads())


@pytest.mark.parametrize("d", [1, 16, 40, 64, 100, 128, 129, 200, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_head_dims(d, causal):
    # up to d = 128 four lanes share a row, beyond it sixteen (16-row workgroups)
    q, k, v, do, kl = make(1, 2, 150, 130, seed=d + 3, d=d, dtype=torch.float32)
    run_and_check(q, k, v, do, kl, causal, what=f"f32 d={d}")


@pytest.mark.parametrize("d", [64, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_key_lens_ragged(causal, d):
    q, k, v, do, kl = make(2, 3, 97, 211, seed=23, key_lens=[150, 0], d=d, dtype=torch.float32)
    run_and_check(q, k, v, do, kl, causal, what=f"f32 key_lens d={d}")
    q, k, v, do, kl = make(1, 2, 211, 97, seed=24, d=d, dtype=torch.float32)
    run_and_check(q, k, v, do, kl, causal, scale=0.2, what=f"f32 N > Nk d={d}")
