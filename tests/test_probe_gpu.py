"""GPU checks of the measurement probes of include/fa_probe.h: the streaming
read touches every byte exactly once (its XOR checksum equals the host's), the
streaming copy reproduces its source byte for byte and writes nothing past its
end, and the matrix-core stream really executes its products (its sums are
finite, nonzero and grow linearly with the iteration count)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_forward_online_amd as fa
from gpu_common import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    fa.load_library()
    yield
    torch.cuda.synchronize()


def host_xor(buf: torch.Tensor) -> int:
    words = buf.cpu().view(torch.int32).numpy().view(np.uint32)
    return int(np.bitwise_xor.reduce(words)) if words.size else 0


@pytest.mark.parametrize("nbytes,blocks", [(0, 3), (16, 1), (16 * 1000 + 16 * 7, 5),
                                           (64 << 20, 2048), ((64 << 20) + 48, 7)])
def test_probe_read_checksum(nbytes, blocks):
    g = torch.Generator(device="cpu").manual_seed(nbytes % 9973)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g).to(DEV)
    say(f"[gpu] fa_probe_read bytes={nbytes} blocks={blocks}")
    sink = fa.probe_read(buf, blocks=blocks)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    assert got == host_xor(buf)


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (16 * 1000 + 16 * 7, 5), (64 << 20, 2048),
                                           ((64 << 20) + 48, 7), (1 << 20, 3000)])
def test_probe_copy_reproduces_source(nbytes, blocks):
    g = torch.Generator(device="cpu").manual_seed(nbytes % 7919)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g).to(DEV)
    big = torch.full((nbytes // 4 + 64,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    dst = big[: nbytes // 4]
    say(f"[gpu] fa_probe_copy bytes={nbytes} blocks={blocks}")
    fa.probe_copy(src, dst, blocks=blocks)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert bool((big[nbytes // 4:] == 0x5A5A5A5A).all())


def test_probe_mfma_executes_every_product():
    say("[gpu] fa_probe_mfma blocks=8 iters=100 / 200")
    s1 = fa.probe_mfma(8, 100).double().cpu()
    s2 = fa.probe_mfma(8, 200).double().cpu()
    torch.cuda.synchronize()
    assert torch.isfinite(s1).all() and torch.isfinite(s2).all()
    assert (s1 != 0).float().mean() > 0.99
    # the accumulators grow by the same products every round: twice the rounds,
    # twice the sums (up to fp32 rounding of the running sums)
    assert torch.allclose(s2, 2 * s1, rtol=1e-3, atol=1e-3 * float(s1.abs().max()))
