"""The decode entry point that allocates nothing (fa_decode_splitkv_noalloc)
against the workspace entry point fa_decode_splitkv, through the C ABI: the
same kernels over the same partial-state layout, so the outputs must agree bit
for bit; both are also checked against the fp64 oracle.  Two calls in a row,
the second smaller than the first, so the second reads only what it wrote
into the shared per-GPU scratch."""
import numpy as np
import pytest
import torch

import attention_forward_online_amd as fa
import oracle
from attention_forward_online_amd.synth import random_case
from gpu_common import compare, say, to_host

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (B, H, Nk, d, splits, dtype, key_lens): the first fills 17.0 MB of the scratch
# (the decode workload's partials: 64 x 32 heads x 16 splits x 130 floats), the
# second a few KB, with an empty and a one-key batch
CASES = [(64, 32, 2048, 128, 16, torch.bfloat16, None),
         (3, 2, 700, 64, 5, torch.float32, [0, 1, 699])]


def test_noalloc_decode_equals_workspace_decode_two_calls():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    fa.load_library()
    for B, H, Nk, d, S, dt, kl in CASES:
        need = fa.fa_decode_workspace_bytes(B, H, d, S)
        assert need <= fa.fa_decode_scratch_bytes()
        inp = random_case(B, H, 1, Nk, d, dt, seed=B + Nk, device=DEV, key_lens=kl)
        q, k, v, klt = inp["q"], inp["k"], inp["v"], inp["key_lens"]
        say(f"[gpu] fa_decode_splitkv_noalloc B={B} H={H} Nk={Nk} d={d} splits={S} {dt} key_lens={kl} "
            f"({need} scratch bytes)")
        o_ws = torch.full_like(q, float("nan"))
        l_ws = torch.full((B, H, 1), float("nan"), device=DEV)
        ws = torch.empty(need // 4, device=DEV)
        fa.fa_decode_splitkv(q, k, v, o_ws, l_ws, S, ws, key_lens=klt)
        o_na = torch.full_like(q, float("nan"))
        l_na = torch.full((B, H, 1), float("nan"), device=DEV)
        fa.fa_decode_splitkv_noalloc(q, k, v, o_na, l_na, S, key_lens=klt)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws), "O differs from the workspace entry point"
        assert torch.equal(l_na, l_ws), "LSE differs from the workspace entry point"
        O_ref, L_ref = oracle.attention(to_host(q), to_host(k), to_host(v),
                                        scale=float(np.float32(1 / np.sqrt(d))), key_lens=kl)
        eo, el = compare(o_na, l_na, O_ref, L_ref, dt, "noalloc decode")
        say(f"    bit-identical to the workspace call; vs oracle max|dO|={eo:.2e} max|dLSE|={el:.2e}")
        del inp, q, k, v, ws
        torch.cuda.empty_cache()
