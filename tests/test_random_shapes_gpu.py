"""Seeded random-shape sweep against the fp64 oracle: the bf16 prefill forward
and backward, the fp32 forward and backward at random head dims, and the
split-KV decode (bf16 and fp32 at d = 64, 128; fp32 at random widths).
Query and key lengths from 1 to 700 (so workgroups hold partial query blocks,
waves with no rows, and odd and even tile counts), causal or not, with or
without per-batch key lengths (including 0 and values past Nk).  Same
tolerances as the fixed-shape tests (bf16 forward 2e-2 on O, 1e-3 on LSE; fp32
1e-5 on both; backward 8e-3 of the largest gradient entry + 1e-3, fp32
backward 2e-5 of it + 1e-6), and rows or
keys that see nothing must be exactly zero."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_forward_online_amd as fa
import oracle
from attention_forward_online_amd.synth import random_case
from gpu_common import compare, forward_and_check, say, to_host
from test_backward_gpu import make, run_and_check

pytestmark = pytest.mark.gpu
DEV = "cuda"


def draw(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 4))
    N = int(rng.integers(1, 701))
    Nk = int(rng.integers(1, 701))
    causal = bool(rng.integers(0, 2))
    key_lens = None
    if rng.random() < 0.5:
        key_lens = [int(x) for x in rng.integers(-2, Nk + 40, size=B)]
        key_lens[int(rng.integers(0, B))] = int(rng.choice([0, Nk, int(rng.integers(1, Nk + 1))]))
    return B, H, N, Nk, causal, key_lens


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seed", list(range(12)))
def test_forward_random_shape(d, seed):
    B, H, N, Nk, causal, kl = draw(1000 * d + seed)
    inp = random_case(B, H, N, Nk, d, torch.bfloat16, seed=seed, device=DEV, key_lens=kl)
    forward_and_check(inp, causal, what=f"random shape seed {seed}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seed", list(range(6)))
def test_backward_random_shape(d, seed):
    B, H, N, Nk, causal, kl = draw(2000 * d + seed)
    q, k, v, do, klt = make(B, H, N, Nk, seed=seed + 50, key_lens=kl, d=d)
    say(f"    random backward seed {seed}")
    run_and_check(q, k, v, do, klt, causal, what=f"random backward seed {seed}")


@pytest.mark.parametrize("seed", list(range(10)))
def test_f32_forward_random_shape(seed):
    B, H, N, Nk, causal, kl = draw(3000 + seed)
    d = int(np.random.default_rng(seed).integers(1, 257))
    inp = random_case(B, H, N, Nk, d, torch.float32, seed=seed, device=DEV, key_lens=kl)
    forward_and_check(inp, causal, what=f"random fp32 shape seed {seed} d={d}")


@pytest.mark.parametrize("seed", list(range(8)))
def test_decode_random_shape(seed):
    rng = np.random.default_rng(4000 + seed)
    B, H = int(rng.integers(1, 9)), int(rng.integers(1, 5))
    Nk = int(rng.integers(0, 5000))
    d = int(rng.choice([64, 128]))
    S = int(rng.integers(1, 65))
    dtype = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    kl = None
    if rng.random() < 0.5:
        kl = [int(x) for x in rng.integers(-2, Nk + 40, size=B)]
    inp = random_case(B, H, 1, Nk, d, dtype, seed=seed, device=DEV, key_lens=kl)
    q, k, v, klt = inp["q"], inp["k"], inp["v"], inp["key_lens"]
    say(f"[gpu] decode random seed {seed}: B={B} H={H} Nk={Nk} d={d} {dtype} splits={S} key_lens={kl}")
    o, lse = fa.decode(q, k, v, num_splits=S, key_lens=klt)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(to_host(q), to_host(k), to_host(v),
                                    scale=float(np.float32(1 / np.sqrt(d))), key_lens=kl)
    compare(o, lse, O_ref, L_ref, dtype, f"decode random seed {seed}")


@pytest.mark.parametrize("seed", list(range(6)))
def test_f32_backward_random_shape(seed):
    B, H, N, Nk, causal, kl = draw(5000 + seed)
    d = int(np.random.default_rng(5000 + seed).integers(1, 257))
    q, k, v, do, klt = make(B, H, N, Nk, seed=seed + 70, key_lens=kl, d=d, dtype=torch.float32)
    say(f"    random fp32 backward seed {seed} d={d}")
    run_and_check(q, k, v, do, klt, causal, what=f"random fp32 backward seed {seed} d={d}")


@pytest.mark.parametrize("seed", list(range(6)))
def test_f32_decode_random_width(seed):
    rng = np.random.default_rng(6000 + seed)
    B, H = int(rng.integers(1, 9)), int(rng.integers(1, 5))
    Nk = int(rng.integers(0, 5000))
    d = int(rng.integers(1, 257))
    S = int(rng.integers(1, 65))
    kl = None
    if rng.random() < 0.5:
        kl = [int(x) for x in rng.integers(-2, Nk + 40, size=B)]
    inp = random_case(B, H, 1, Nk, d, torch.float32, seed=seed, device=DEV, key_lens=kl)
    q, k, v, klt = inp["q"], inp["k"], inp["v"], inp["key_lens"]
    say(f"[gpu] fp32 decode random seed {seed}: B={B} H={H} Nk={Nk} d={d} splits={S} key_lens={kl}")
    o, lse = fa.decode(q, k, v, num_splits=S, key_lens=klt)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(to_host(q), to_host(k), to_host(v),
                                    scale=float(np.float32(1 / np.sqrt(d))), key_lens=kl)
    compare(o, lse, O_ref, L_ref, torch.float32, f"fp32 decode random seed {seed} d={d}")
