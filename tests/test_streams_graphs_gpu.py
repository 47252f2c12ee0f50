"""Every entry point on a non-default stream, and captured into a HIP graph
(torch.cuda.graph) that is replayed several times with new inputs copied into
its static buffers, eager work and synchronisations in between.  Each result
must equal, bit for bit, the eager call on the same inputs (same kernels, same
order of operations).  The one-pass softmax resets its ticket counter with a
kernel, so replays need no memset node."""
from __future__ import annotations

import pytest
import torch

import attention_forward_online_amd as fa
from attention_forward_online_amd import synth
from gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def same(a, b):
    return torch.equal(bits(a), bits(b))


def fresh(shape, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(dtype)


def test_side_stream_matches_default_stream():
    inp = synth.random_case(2, 4, 300, 300, 64, torch.bfloat16, seed=1, device=DEV)
    say("[gpu] streams: forward / decode / softmax / backward on a side stream")
    o0, l0 = fa.attention(inp["q"], inp["k"], inp["v"], causal=True)
    x = fresh((64, 70001), torch.float32, 2)
    y0, s0 = fa.softmax(x)
    do = fresh(inp["q"].shape, torch.bfloat16, 3)
    g0 = fa.attention_backward(inp["q"], inp["k"], inp["v"], o0, l0, do, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o1, l1 = fa.attention(inp["q"], inp["k"], inp["v"], causal=True)
        y1, s1 = fa.softmax(x)
        g1 = fa.attention_backward(inp["q"], inp["k"], inp["v"], o1, l1, do, causal=True)
    side.synchronize()
    assert same(o0, o1) and same(l0, l1) and same(y0, y1) and same(s0, s1)
    assert all(same(a, b) for a, b in zip(g0, g1))


def test_bound_launchers_match_the_checked_calls():
    """bind_forward / bind_backward: bound once, run twice with new inputs copied
    into the same buffers (and once on a side stream bound there), each result
    bit-identical to the checked call on the same inputs."""
    B, H, N, d = 2, 3, 257, 64
    q = torch.empty((B, H, N, d), device=DEV, dtype=torch.bfloat16)
    k, v, do = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), device=DEV, dtype=torch.float32)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N) // 4, device=DEV, dtype=torch.float32)
    kl = torch.tensor([190, 257], dtype=torch.int32, device=DEV)
    fwd = fa.bind_forward(q, k, v, o, lse, causal=True, key_lens=kl)
    bwd = fa.bind_backward(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True, key_lens=kl)
    for r in range(2):
        say(f"[gpu] bound launchers: round {r}")
        for i, t in enumerate((q, k, v, do)):
            t.copy_(fresh(t.shape, t.dtype, 300 + 10 * r + i))
        fwd()
        bwd()
        torch.cuda.synchronize()
        oe, le = fa.attention(q, k, v, causal=True, key_lens=kl)
        ge = fa.attention_backward(q, k, v, oe, le, do, causal=True, key_lens=kl)
        torch.cuda.synchronize()
        assert same(o, oe) and same(lse, le), f"round {r}: bound forward differs"
        assert all(same(a, b) for a, b in zip((dq, dk, dv), ge)), f"round {r}: bound backward differs"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o.zero_()
    with torch.cuda.stream(side):
        fa.bind_forward(q, k, v, o, lse, causal=True, key_lens=kl)()
    side.synchronize()
    assert same(o, oe) and same(lse, le), "bound forward on a side stream differs"


def capture(fn):
    """Warm up on a side stream (torch's rule for capture), then capture fn."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def test_graph_replays_forward_and_decode():
    B, H, N, d = 2, 4, 333, 128
    q = torch.empty((B, H, N, d), device=DEV, dtype=torch.bfloat16)
    k, v = torch.empty_like(q), torch.empty_like(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=DEV, dtype=torch.float32)
    qd = torch.empty((B, H, 1, d), device=DEV, dtype=torch.bfloat16)
    od = torch.empty_like(qd)
    ld = torch.empty((B, H, 1), device=DEV, dtype=torch.float32)
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, d, 8) // 4, device=DEV, dtype=torch.float32)
    # a non-causal call on this small grid runs the key-split kernel; key length 0
    # for one batch takes the early exit
    o2, lse2 = torch.empty_like(q), torch.empty_like(lse)
    kl = torch.tensor([0, 201], dtype=torch.int32, device=DEV)
    # a small fp32 call runs the key-ways fp32 kernel
    qf = torch.empty((1, 2, 77, 64), device=DEV, dtype=torch.float32)
    kf, vf, of = torch.empty_like(qf), torch.empty_like(qf), torch.empty_like(qf)
    lf = torch.empty((1, 2, 77), device=DEV, dtype=torch.float32)
    # an fp32 decode of a width other than 64 and 128 (rows read element by element)
    qg = torch.empty((2, 3, 1, 101), device=DEV, dtype=torch.float32)
    kg = torch.empty((2, 3, 900, 101), device=DEV, dtype=torch.float32)
    vg, og = torch.empty_like(kg), torch.empty_like(qg)
    lg = torch.empty((2, 3, 1), device=DEV, dtype=torch.float32)
    wsg = torch.empty(fa.fa_decode_workspace_bytes(2, 3, 101, 5) // 4, device=DEV, dtype=torch.float32)
    for t in (q, k, v, qd, qf, kf, vf, qg, kg, vg):
        t.copy_(fresh(t.shape, t.dtype, 0))

    def step():
        fa.fa_forward(q, k, v, o, lse, causal=True)
        fa.fa_decode_splitkv(qd, k, v, od, ld, 8, ws)
        fa.fa_forward(q, k, v, o2, lse2, causal=False, key_lens=kl)
        fa.fa_forward(qf, kf, vf, of, lf, causal=False)
        fa.fa_decode_splitkv(qg, kg, vg, og, lg, 5, wsg)

    graph = capture(step)
    for r in range(3):
        say(f"[gpu] graphs: forward + decode replay {r}")
        for i, t in enumerate((q, k, v, qd, qf, kf, vf, qg, kg, vg)):
            t.copy_(fresh(t.shape, t.dtype, 10 * r + i + 1))
        graph.replay()
        torch.cuda.synchronize()
        oe, le = fa.attention(q, k, v, causal=True)
        ode, lde = fa.decode(qd, k, v, num_splits=8)
        oe2, le2 = fa.attention(q, k, v, causal=False, key_lens=kl)
        oef, lef = fa.attention(qf, kf, vf, causal=False)
        oeg, leg = fa.decode(qg, kg, vg, num_splits=5)
        torch.cuda.synchronize()
        assert same(o, oe) and same(lse, le), f"replay {r}: forward differs from eager"
        assert same(od, ode) and same(ld, lde), f"replay {r}: decode differs from eager"
        assert same(o2, oe2) and same(lse2, le2), f"replay {r}: key-split forward differs from eager"
        assert same(of, oef) and same(lf, lef), f"replay {r}: fp32 forward differs from eager"
        assert same(og, oeg) and same(lg, leg), f"replay {r}: fp32 d=101 decode differs from eager"


@pytest.mark.parametrize("cols", [3000, 70001, 262144])
def test_graph_replays_softmax(cols):
    rows = 48
    x = torch.empty((rows, cols), device=DEV, dtype=torch.float32)
    y = torch.empty_like(x)
    lse = torch.empty(rows, device=DEV, dtype=torch.float32)
    nb = fa.fa_softmax_workspace_bytes(rows, cols, torch.float32)
    ws = torch.empty(max(nb, 16) // 4, device=DEV, dtype=torch.float32)
    x.copy_(fresh(x.shape, x.dtype, 5))
    graph = capture(lambda: fa.fa_softmax(x, y, lse, ws))
    for r in range(4):
        say(f"[gpu] graphs: softmax cols={cols} replay {r}")
        x.copy_(fresh(x.shape, x.dtype, 100 + r) * (1 + r))
        graph.replay()
        torch.cuda.synchronize()
        ye, le = fa.softmax(x)
        torch.cuda.synchronize()
        assert same(y, ye) and same(lse, le), f"replay {r}: softmax differs from eager"


@pytest.mark.parametrize("d,dtype", [(64, torch.bfloat16), (128, torch.bfloat16), (200, torch.float32)])
def test_graph_replays_backward(d, dtype):
    # d = 128: the paired dK/dV kernel (P through two LDS buffers by tile
    # parity); fp32 d = 200: sixteen lanes per row
    B, H, N = 1, 4, 200
    q = torch.empty((B, H, N, d), device=DEV, dtype=dtype)
    k, v, do = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), device=DEV, dtype=torch.float32)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N) // 4, device=DEV, dtype=torch.float32)
    for t in (q, k, v, do):
        t.copy_(fresh(t.shape, t.dtype, 7))

    def step():
        fa.fa_forward(q, k, v, o, lse, causal=True)
        fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True)

    graph = capture(step)
    for r in range(3):
        say(f"[gpu] graphs: forward + backward d={d} {dtype} replay {r}")
        for i, t in enumerate((q, k, v, do)):
            t.copy_(fresh(t.shape, t.dtype, 50 + 10 * r + i))
        graph.replay()
        torch.cuda.synchronize()
        oe, le = fa.attention(q, k, v, causal=True)
        ge = fa.attention_backward(q, k, v, oe, le, do, causal=True)
        torch.cuda.synchronize()
        assert same(o, oe) and same(lse, le)
        assert all(same(a, b) for a, b in zip((dq, dk, dv), ge)), f"replay {r}: backward differs"
