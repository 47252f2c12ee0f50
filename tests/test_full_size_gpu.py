"""GPU parity at the full sizes of the five workloads: every output element of
the HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs, in the launch configuration bench.py times.

Tolerances (max |GPU - oracle|): bf16 2e-2 on O and 1e-3 on LSE, fp32 1e-5 on
both; rows without a visible key exactly O = 0, LSE = -inf; no NaN anywhere.
The oracle runs threaded over rows on the host's cores (the 8192-long causal
prefill is about 2.7e11 fp64 multiply-adds)."""
import os

import numpy as np
import pytest
import torch

import attention_forward_online_amd as fa
import oracle
from attention_forward_online_amd.synth import WORKLOADS, make_inputs
from gpu_common import compare, say, to_host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def host_threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, 32))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    fa.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["tiny_f32_b1h1_n256_d64", "causal_bf16_b4h16_n2048_d64",
                                  "causal_bf16_b1h32_n8192_d128", "masked_bf16_b2h8_n4096_d128"])
def test_prefill_workload_every_row(name):
    w = WORKLOADS[name]
    inp = make_inputs(w, device=DEV)
    q, k, v, kl = inp["q"], inp["k"], inp["v"], inp["key_lens"]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.N), float("nan"), device=DEV)
    say(f"[gpu] fa_forward {name} (every row) key_lens={None if kl is None else kl.tolist()}")
    fa.fa_forward(q, k, v, o, lse, causal=w.causal, key_lens=kl)
    torch.cuda.synchronize()
    klh = None if kl is None else kl.tolist()
    O_ref, L_ref = oracle.attention(to_host(q), to_host(k), to_host(v), scale=float(np.float32(w.scale)),
                                    causal=w.causal, key_lens=klh, nthreads=host_threads())
    eo, el = compare(o, lse, O_ref, L_ref, q.dtype, name)
    say(f"    {w.B * w.H * w.N} rows: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    if klh is not None:
        # the batch without keys: every row exactly O = 0, LSE = -inf
        for b, n in enumerate(klh):
            if n == 0:
                assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))


def test_decode_workload_every_head():
    w = WORKLOADS["decode_bf16_b64h32_nk16384_d128"]
    inp = make_inputs(w, device=DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, 1), float("nan"), device=DEV)
    ws = torch.empty(fa.fa_decode_workspace_bytes(w.B, w.H, w.d, w.num_splits) // 4, device=DEV)
    say(f"[gpu] fa_decode_splitkv {w.name} (every head)")
    fa.fa_decode_splitkv(q, k, v, o, lse, w.num_splits, ws)
    torch.cuda.synchronize()
    eo = el = 0.0
    for b in range(w.B):   # one batch at a time bounds host memory (256 MiB of K and V each)
        O_ref, L_ref = oracle.attention(to_host(q[b:b + 1]), to_host(k[b:b + 1]), to_host(v[b:b + 1]),
                                        scale=float(np.float32(w.scale)), nthreads=host_threads())
        e1, e2 = compare(o[b:b + 1], lse[b:b + 1], O_ref, L_ref, q.dtype, f"{w.name} b={b}")
        eo, el = max(eo, e1), max(el, e2)
    say(f"    {w.B * w.H} heads: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
