"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Tolerances (max |GPU - oracle|): fp32 1e-5 on O and LSE;
bf16 2e-2 on O and 1e-3 on LSE.  Rows without a visible key must be exactly
O = 0, LSE = -inf; no NaN anywhere."""
import numpy as np
import pytest
import torch

import attention_forward_online_amd as fa
import oracle
from attention_forward_online_amd.synth import WORKLOADS, make_inputs, random_case
from gpu_common import compare, forward_and_check, sample_rows, say, to_host

pytestmark = pytest.mark.gpu
DEV = "cuda"
F32, BF16 = torch.float32, torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    fa.load_library()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ fp32 path
def test_f32_tiny_workload():
    w = WORKLOADS["tiny_f32_b1h1_n256_d64"]
    inp = make_inputs(w, device=DEV)
    eo, el, *_ = forward_and_check(inp, w.causal, what=w.name)
    say(f"    max|dO|={eo:.2e} max|dLSE|={el:.2e}")


@pytest.mark.parametrize("N,Nk,d", [(6, 6, 4), (10, 7, 8), (1, 1, 2), (5, 13, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_page_tile_shapes(N, Nk, d, causal):
    inp = random_case(1, 1, N, Nk, d, F32, seed=3, device=DEV)
    forward_and_check(inp, causal, what="page shape")


@pytest.mark.parametrize("d", [1, 3, 16, 17, 64, 100, 128, 200, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_head_dims_ragged(d, causal):
    inp = random_case(2, 2, 70, 97, d, F32, seed=d, device=DEV, key_lens=[50, 97])
    forward_and_check(inp, causal, what="f32 ragged")


@pytest.mark.parametrize("d", [64, 100, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_large_grid(d, causal):
    # 2 x 32 heads of 256 rows: enough 64-row workgroups for the 4-lanes-per-row
    # kernel (small grids take the 16-lane one); sampled rows of 8 heads
    inp = random_case(2, 32, 256, 256, d, F32, seed=d + 7, device=DEV, key_lens=[256, 201])
    rows = sample_rows(2, 32, 256, per_head=8, seed=d, bh_limit=8)
    forward_and_check(inp, causal, what="f32 large grid", rows=rows)


def test_f32_key_lens_edges():
    inp = random_case(5, 1, 40, 33, 32, F32, seed=9, device=DEV, key_lens=[0, 1, 32, 33, 1000])
    forward_and_check(inp, False, what="f32 key_lens")
    inp["key_lens"] = torch.tensor([-5, 2, 31, 7, 0], dtype=torch.int32, device=DEV)
    forward_and_check(inp, True, what="f32 key_lens causal")


# ------------------------------------------------------------------ bf16 prefill
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,Nk", [(300, 333), (128, 128), (1, 1), (1, 200), (200, 390), (390, 200),
                                  (257, 64), (64, 1)])
def test_bf16_ragged(d, causal, N, Nk):
    inp = random_case(2, 3, N, Nk, d, BF16, seed=N + Nk, device=DEV)
    forward_and_check(inp, causal, what="bf16 ragged")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_key_lens(d, causal):
    # 0 (fully masked batch), 1, tile edges, beyond Nk (clamped) and negative (clamped to 0)
    kl = [0, 1, 63, 64, 65, 500, -3, 129]
    inp = random_case(8, 2, 130, 300, d, BF16, seed=d, device=DEV, key_lens=kl)
    forward_and_check(inp, causal, what="bf16 key_lens")


@pytest.mark.parametrize("B,H,N,Nk,d", [(64, 2, 70, 150, 64), (64, 8, 300, 200, 128),
                                          (3, 5, 257, 300, 64), (65, 1, 64, 64, 64),
                                          (200, 2, 70, 150, 128), (1024, 1, 16, 40, 64),
                                          (1025, 1, 16, 40, 64), (96, 8, 64, 100, 64)])
def test_bf16_key_length_launch_order(B, H, N, Nk, d):
    # non-causal grids with key lengths go out batch by batch: up to 64 batches in
    # descending order of visible keys (each workgroup ranks all batches), up to 1024
    # with the batches that have keys first (per-64 masks), beyond that in the plain
    # order: every (head, block) must be computed exactly once.  Key lengths with ties,
    # 0, Nk, past Nk and negative; 128 blocks (key split), 1536 blocks, heads not a
    # multiple of 8.  Outputs start as NaN, so a block left out or written twice with
    # the wrong rows shows.  B = 96: more than 64 batches, none empty (the head-per-XCD
    # order then applies).
    rng = np.random.default_rng(B * 1000 + N)
    choices = [1, 37, Nk // 2, Nk, Nk + 9] if B == 96 else [0, 1, 37, Nk // 2, Nk // 2, Nk, Nk + 9, -3]
    kl = [int(x) for x in rng.choice(choices, size=B)]
    inp = random_case(B, H, N, Nk, d, BF16, seed=B + d, device=DEV, key_lens=kl)
    o = torch.full_like(inp["q"], float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    say(f"[gpu] fa_forward key-length order B={B} H={H} N={N} Nk={Nk} d={d} key_lens={kl}")
    fa.fa_forward(inp["q"], inp["k"], inp["v"], o, lse, causal=False, key_lens=inp["key_lens"])
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(to_host(inp["q"]), to_host(inp["k"]), to_host(inp["v"]),
                                    scale=float(np.float32(1.0 / np.sqrt(d))), key_lens=kl)
    compare(o, lse, O_ref, L_ref, BF16, f"key-length order B={B}")


@pytest.mark.parametrize("kl", [[0, 300, 300, 0], [500, 300, 200, 100], [500, 300, 200, 0],
                                [0, 0, 0, 0], [600, 1, 64, 65]])
def test_bf16_key_length_order_one_to_two_blocks_per_cu(kl):
    # d = 128, non-causal, key lengths, between one and two blocks per CU (the
    # masked workload's regime): batches with keys first in the launch order,
    # batches without keys (O = 0, LSE = -inf) after them, equal and unequal tile
    # counts side by side.  Outputs start as NaN.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, H, Nk, d = 4, 16, 600, 128
    n_qt = (3 * cus) // (2 * B * H)
    N = n_qt * 128 - 28
    assert cus < B * H * n_qt <= 2 * cus
    inp = random_case(B, H, N, Nk, d, BF16, seed=sum(kl) + 3, device=DEV, key_lens=kl)
    o = torch.full_like(inp["q"], float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    say(f"[gpu] fa_forward key-length order, 1-2 blocks per CU B={B} H={H} N={N} Nk={Nk} key_lens={kl}")
    fa.fa_forward(inp["q"], inp["k"], inp["v"], o, lse, causal=False, key_lens=inp["key_lens"])
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(to_host(inp["q"]), to_host(inp["k"]), to_host(inp["v"]),
                                    scale=float(np.float32(1.0 / np.sqrt(d))), key_lens=kl)
    compare(o, lse, O_ref, L_ref, BF16, f"key-length order, 1-2 blocks per CU {kl}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("extra_heads", [0, 1])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_key_split_grid_boundary(d, extra_heads, causal):
    # a grid of at most one query block per CU runs each block's keys in two halves
    # merged at the end; one more head per batch puts the same inputs on the unsplit
    # path.  Key lengths: none (the block leaves at once), one tile split 1 / 0, tile
    # edges, odd tile counts, full; causal with Nk > N puts the diagonal in the second half.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, N, Nk = 8, 100, 300
    H = cus // B + extra_heads
    kl = [0, 1, 64, 65, 129, 200, 255, 300]
    inp = random_case(B, H, N, Nk, d, BF16, seed=41 + d, device=DEV, key_lens=kl)
    rows = sample_rows(B, H, N, per_head=8, seed=d, bh_limit=40)
    rows += [b * H * N + i for b in range(B) for i in (0, N - 1)]
    forward_and_check(inp, causal, what=f"bf16 {B * H} blocks vs {cus} CUs", rows=sorted(set(rows)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_largest_slice(d, causal):
    # the largest K/V slice per (batch, head) the library accepts: Nk * d * 2 bytes just
    # under 2^31 (its 32-bit buffer offsets); a key more is rejected before any launch
    Nk = ((1 << 31) - 256) // (2 * d)
    N = 130
    inp = random_case(1, 1, N, Nk, d, BF16, seed=7 + d, device=DEV)
    rows = [0, 1, 63, 64, 127, 128, N - 1]
    forward_and_check(inp, causal, what=f"bf16 largest slice Nk={Nk}", rows=rows)
    k1 = torch.empty(1, 1, Nk + 1, d, dtype=BF16, device=DEV)
    o = torch.empty_like(inp["q"])
    lse = torch.empty(1, 1, N, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError, match="FA_ERR_INVALID_ARG"):
        fa.fa_forward(inp["q"], k1, k1, o, lse, causal=causal)
    del inp, k1
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("sigma", [3.0, 12.0])
def test_bf16_high_dynamic_range(d, sigma):
    inp = random_case(2, 4, 256, 640, d, BF16, seed=17, device=DEV, q_sigma=sigma, key_lens=[640, 333])
    forward_and_check(inp, False, what=f"bf16 q~N(0,{sigma ** 2:g})")
    forward_and_check(inp, True, what=f"bf16 q~N(0,{sigma ** 2:g}) causal")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("slope", [0.02, 0.3, -0.3, 3.0])
def test_bf16_score_ramps(d, slope):
    # scores that rise (or fall) steadily along the keys: the running max moves
    # by less than, or by much more than, a rescale rule tolerates per tile
    # (threshold 8 in log2 units, guard weights below 2^32);
    # rows of several batches see different key lengths, one of them none
    B, H, N, Nk = 3, 2, 200, 700
    g = torch.Generator().manual_seed(11)
    q = torch.zeros(B, H, N, d)
    q[..., 0] = 1.0 + 0.1 * torch.rand(B, H, N, generator=g)
    k = 0.05 * torch.randn(B, H, Nk, d, generator=g)
    k[..., 0] += slope * torch.arange(Nk, dtype=torch.float32)
    v = torch.randn(B, H, Nk, d, generator=g)
    inp = {"q": q.to(BF16).to(DEV), "k": k.to(BF16).to(DEV), "v": v.to(BF16).to(DEV),
           "key_lens": torch.tensor([700, 0, 333], dtype=torch.int32, device=DEV)}
    forward_and_check(inp, False, scale=1.0 / 8, what=f"ramp slope {slope}")
    forward_and_check(inp, True, scale=1.0 / 8, what=f"ramp slope {slope} causal")


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_no_keys_gives_zero_and_neg_inf(dtype):
    q = torch.randn(2, 3, 40, 64, device=DEV).to(dtype)
    k = torch.empty(2, 3, 0, 64, device=DEV, dtype=dtype)
    o = torch.full_like(q, 7.0)
    lse = torch.zeros(2, 3, 40, device=DEV)
    say("[gpu] fa_forward Nk=0")
    fa.fa_forward(q, k, k, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_bf16_deterministic_and_scale():
    inp = random_case(2, 8, 384, 384, 128, BF16, seed=5, device=DEV)
    o1, l1 = fa.attention(inp["q"], inp["k"], inp["v"], causal=True)
    o2, l2 = fa.attention(inp["q"], inp["k"], inp["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    forward_and_check(inp, True, scale=0.37, what="bf16 scale 0.37")


# ------------------------------------------------------------------ decode
def _decode_check(inp, S, what):
    q, k, v, kl = inp["q"], inp["k"], inp["v"], inp["key_lens"]
    say(f"[gpu] fa_decode_splitkv {what} B={q.shape[0]} H={q.shape[1]} Nk={k.shape[2]} "
        f"d={q.shape[3]} {q.dtype} splits={S}")
    o, lse = fa.decode(q, k, v, num_splits=S, key_lens=kl)
    torch.cuda.synchronize()
    d = q.shape[3]
    O_ref, L_ref = oracle.attention(to_host(q), to_host(k), to_host(v),
                                    scale=float(np.float32(1 / np.sqrt(d))),
                                    key_lens=None if kl is None else to_host(kl).tolist())
    return compare(o, lse, O_ref, L_ref, q.dtype, what) + (o, lse)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", [1, 2, 16, 37])
def test_decode_small(dtype, d, S):
    inp = random_case(3, 2, 1, 1000, d, dtype, seed=S, device=DEV)
    _decode_check(inp, S, "decode small")


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_decode_key_lens_and_empty(dtype):
    inp = random_case(5, 2, 1, 700, 128, dtype, seed=2, device=DEV, key_lens=[0, 1, 699, 5000, 17])
    _decode_check(inp, 16, "decode key_lens")
    inp = random_case(2, 2, 1, 0, 64, dtype, seed=2, device=DEV)
    _decode_check(inp, 4, "decode Nk=0")


@pytest.mark.parametrize("d", [1, 3, 16, 17, 40, 100, 129, 200, 256])
@pytest.mark.parametrize("S", [1, 16])
def test_decode_f32_widths(d, S):
    # fp32 rows of widths other than 64 and 128 (the lanes past d hold zeros;
    # widths that are not a multiple of 4 are read element by element), with a
    # key length, an empty batch and a short one; the result equals the fp32
    # forward's with one query to rounding
    inp = random_case(3, 2, 1, 700, d, F32, seed=d + S, device=DEV, key_lens=[700, 0, 333])
    _, _, o, lse = _decode_check(inp, S, f"decode f32 d={d}")
    o_f, l_f = fa.attention(inp["q"], inp["k"], inp["v"], key_lens=inp["key_lens"])
    torch.cuda.synchronize()
    assert torch.allclose(o, o_f, rtol=0, atol=2e-6)
    assert torch.equal(torch.isinf(lse), torch.isinf(l_f))
    fin = torch.isfinite(l_f)
    assert torch.allclose(lse[fin], l_f[fin], rtol=0, atol=5e-6)


def test_decode_matches_forward_and_split_invariance():
    inp = random_case(4, 4, 1, 3000, 128, F32, seed=8, device=DEV, key_lens=[3000, 2047, 1, 512])
    q, k, v, kl = inp["q"], inp["k"], inp["v"], inp["key_lens"]
    o_f, l_f = fa.attention(q, k, v, key_lens=kl)
    outs = [fa.decode(q, k, v, num_splits=S, key_lens=kl) for S in (1, 2, 4, 16, 64)]
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.allclose(o, o_f, rtol=0, atol=2e-6)
        assert torch.allclose(l, l_f, rtol=0, atol=5e-6)
    o1, l1 = fa.decode(q, k, v, num_splits=16, key_lens=kl)
    torch.cuda.synchronize()
    assert torch.equal(o1, outs[3][0]) and torch.equal(l1, outs[3][1])


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_decode_largest_slice(dtype):
    # the largest K/V slice per (batch, head) the decode accepts (Nk * d * element size
    # just under 2^31), over 16 splits, with and without a key length cutting it
    d = 128
    esz = 4 if dtype == F32 else 2
    Nk = ((1 << 31) - 256) // (esz * d)
    inp = random_case(2, 1, 1, Nk, d, dtype, seed=3, device=DEV, key_lens=[Nk, Nk // 3 + 5])
    _decode_check(inp, 16, f"decode largest slice Nk={Nk}")
    _decode_check(inp, 1, f"decode largest slice Nk={Nk}, one split")
    del inp
    torch.cuda.empty_cache()


def test_f32_largest_slice():
    # fp32 prefill at the largest accepted slice (Nk * d * 4 bytes just under 2^31)
    d = 64
    Nk = ((1 << 31) - 256) // (4 * d)
    inp = random_case(1, 1, 37, Nk, d, F32, seed=5, device=DEV)
    forward_and_check(inp, False, what=f"f32 largest slice Nk={Nk}", rows=[0, 1, 17, 36])
    forward_and_check(inp, True, what=f"f32 largest slice causal Nk={Nk}", rows=[0, 1, 17, 36])
    del inp
    torch.cuda.empty_cache()


# ------------------------------------------------------------ rescale rules
def _spike_case(B, H, N, Nk, d, seed, first_low):
    # scores ~ N(0, 1/8) plus single keys whose score jumps by 200 (far past any
    # weight limit) at positions in the first and the second half of 64-key tiles,
    # and optionally a first tile 1000 below the rest (the reference must move up
    # from there); key lengths cut some batches
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g)
    q[..., 0] = 1.0
    k = 0.25 * torch.randn(B, H, Nk, d, generator=g)
    k[..., 0] = 0.0
    for j in (5, 40, 97, 170, 230):
        if j < Nk:
            k[:, :, j, 0] = 200.0 * (1 + j % 3)
    if first_low:
        k[:, :, :64, 0] = -1000.0
    v = torch.randn(B, H, Nk, d, generator=g)
    return {"q": q.to(BF16).to(DEV), "k": k.to(BF16).to(DEV), "v": v.to(BF16).to(DEV),
            "key_lens": torch.tensor([Nk, 150, 64, 41][:B], dtype=torch.int32, device=DEV)}


@pytest.mark.parametrize("rule", [fa.RESCALE_EAGER, fa.RESCALE_THRESHOLD, fa.RESCALE_GUARD])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_rescale_rules(rule, d, causal):
    # every rule by which the prefill moves its reference max gives the oracle's
    # result: ordinary scores, a high dynamic range, score spikes in either half
    # of a tile and a first tile far below the rest (slow paths of the guard rule)
    fa.testing_set_rescale_rule(rule)
    try:
        inp = random_case(2, 3, 200, 333, d, BF16, seed=d + rule, device=DEV, key_lens=[333, 97])
        forward_and_check(inp, causal, what=f"rule {rule}")
        inp = random_case(2, 2, 160, 300, d, BF16, seed=3 * d + rule, device=DEV, q_sigma=12.0,
                          key_lens=[300, 131])
        forward_and_check(inp, causal, what=f"rule {rule} q~N(0,144)")
        for first_low in (False, True):
            inp = _spike_case(4, 2, 130, 260, d, seed=d + 7 * rule, first_low=first_low)
            forward_and_check(inp, causal, scale=1.0 / 8, what=f"rule {rule} spikes first_low={first_low}")
    finally:
        fa.testing_set_rescale_rule(fa.RESCALE_GUARD)


@pytest.mark.parametrize("B,H,N,Nk,d,causal", [(1, 32, 300, 3000, 128, True), (1, 16, 200, 9000, 64, True),
                                                (2, 16, 130, 4500, 128, False), (1, 8, 64, 16384, 128, True)])
def test_bf16_grouped_head_order(B, H, N, Nk, d, causal):
    # when an XCD's heads stream more K/V than its L2 holds, their blocks go in
    # groups of heads (here groups of 2 and of 1 head): every (head, block) must
    # be computed exactly once; outputs start as NaN
    inp = random_case(B, H, N, Nk, d, BF16, seed=N + Nk + d, device=DEV)
    o = torch.full_like(inp["q"], float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    say(f"[gpu] fa_forward grouped head order B={B} H={H} N={N} Nk={Nk} d={d} causal={causal}")
    fa.fa_forward(inp["q"], inp["k"], inp["v"], o, lse, causal=causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(to_host(inp["q"]), to_host(inp["k"]), to_host(inp["v"]),
                                    scale=float(np.float32(1.0 / np.sqrt(d))), causal=causal)
    compare(o, lse, O_ref, L_ref, BF16, f"grouped head order B={B} H={H} Nk={Nk}")
