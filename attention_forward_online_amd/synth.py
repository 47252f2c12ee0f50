"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both sides of every parity check read the bytes made
here: the HIP library receives them on the device, the fp64 reference receives
a host copy of the very same bytes.

Recipe (per workload, per tensor, per batch index b):
  * a seed derived from (base seed, workload name, tensor name, b) with CRC32;
  * a torch Philox/CPU generator seeded with it, on the device the tensor is
    drawn on (``gen_device``: "cpu" or "cuda");
  * float32 standard normals times sigma, rounded to the storage dtype with
    torch's round-to-nearest-even conversion;
  * key lengths (masked workload only) drawn uniformly from {0..Nk} with a CPU
    generator, and the last batch's length forced to 0 so that one batch has
    only fully masked rows.

The shapes follow the problem statement of the pages: Q and O are [B, H, N, d],
K and V are [B, H, Nk, d], LSE is [B, H, N] (decode: N = 1).

Row softmax workloads (score rows of long-context attention): X is
[rows, cols]; rows are drawn in blocks of rows, each block from its own
derived seed, as sigma-scaled float32 normals rounded to the storage dtype;
row r keeps a valid prefix of length len_r drawn uniformly from {0..cols} and
holds -inf beyond it (the shape of a causal or padding mask), with len_0 =
cols (no masked entry) and the last row's length forced to 0 (fully masked).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int          # query rows per (b, h); 1 for decode
    Nk: int         # keys per (b, h)
    d: int          # head dimension
    dtype: str      # "f32" or "bf16": storage and MFMA operand type
    causal: bool
    q_sigma: float = 1.0
    kv_sigma: float = 1.0
    key_lens: bool = False      # per-batch key lengths (last batch forced to 0)
    decode: bool = False        # one query per sequence, split-KV path
    num_splits: int = 0         # decode only

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def describe(self) -> str:
        kind = "decode" if self.decode else ("causal prefill" if self.causal else "prefill")
        extra = f" splits={self.num_splits}" if self.decode else ""
        extra += " key_lens=[U{0..Nk}, ..., 0]" if self.key_lens else ""
        return (f"{kind} B={self.B} H={self.H} N={self.N} Nk={self.Nk} d={self.d} "
                f"{self.dtype} q~N(0,{self.q_sigma ** 2:g}){extra}")


# The five workloads of the target: a small fp32 case, two causal bf16
# prefills, a one-query split-KV decode and a masked high-dynamic-range prefill.
WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32_b1h1_n256_d64", 1, 1, 256, 256, 64, "f32", False),
        Workload("causal_bf16_b4h16_n2048_d64", 4, 16, 2048, 2048, 64, "bf16", True),
        Workload("causal_bf16_b1h32_n8192_d128", 1, 32, 8192, 8192, 128, "bf16", True),
        Workload("decode_bf16_b64h32_nk16384_d128", 64, 32, 1, 16384, 128, "bf16", False,
                 decode=True, num_splits=16),
        Workload("masked_bf16_b2h8_n4096_d128", 2, 8, 4096, 4096, 128, "bf16", False,
                 q_sigma=3.0, key_lens=True),
    ]
}


def derive_seed(base: int, workload: str, tensor: str, b: int) -> int:
    """Stable 31-bit seed for one (workload, tensor, batch) slice."""
    return zlib.crc32(f"{base}/{workload}/{tensor}/{b}".encode()) & 0x7FFFFFFF


def _generator(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn_slices(shape, sigma: float, dtype: torch.dtype, base_seed: int, workload: str,
                 tensor: str, device: str = "cpu", gen_device: Optional[str] = None) -> torch.Tensor:
    """[B, ...] tensor whose slice b is N(0, sigma^2) from its own derived seed."""
    gen_device = gen_device or ("cuda" if str(device).startswith("cuda") else "cpu")
    out = torch.empty(shape, dtype=dtype, device=device)
    for b in range(shape[0]):
        g = _generator(derive_seed(base_seed, workload, tensor, b), gen_device)
        x = torch.randn(shape[1:], generator=g, device=gen_device, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        out[b].copy_(x.to(dtype))
    return out


def draw_key_lens(B: int, Nk: int, base_seed: int, workload: str) -> torch.Tensor:
    """int32 [B]: uniform on {0..Nk} from the seed; the last batch is forced to 0."""
    g = _generator(derive_seed(base_seed, workload, "key_lens", 0), "cpu")
    kl = torch.randint(0, Nk + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    kl[B - 1] = 0
    return kl


def make_inputs(w: Workload, base_seed: int = 0, device: str = "cpu",
                gen_device: Optional[str] = None) -> dict:
    """Q, K, V (and key_lens or None) for workload ``w`` on ``device``."""
    dt = w.torch_dtype
    q = randn_slices((w.B, w.H, w.N, w.d), w.q_sigma, dt, base_seed, w.name, "q", device, gen_device)
    k = randn_slices((w.B, w.H, w.Nk, w.d), w.kv_sigma, dt, base_seed, w.name, "k", device, gen_device)
    v = randn_slices((w.B, w.H, w.Nk, w.d), w.kv_sigma, dt, base_seed, w.name, "v", device, gen_device)
    kl = draw_key_lens(w.B, w.Nk, base_seed, w.name).to(device) if w.key_lens else None
    return {"q": q, "k": k, "v": v, "key_lens": kl}


def random_case(B, H, N, Nk, d, dtype: torch.dtype, seed: int, device: str = "cpu",
                q_sigma: float = 1.0, key_lens: Optional[list] = None) -> dict:
    """Small ad-hoc case (tests): same recipe, workload name built from the shape."""
    name = f"case_{B}_{H}_{N}_{Nk}_{d}_{dtype}"
    q = randn_slices((B, H, N, d), q_sigma, dtype, seed, name, "q", device)
    k = randn_slices((B, H, Nk, d), 1.0, dtype, seed, name, "k", device)
    v = randn_slices((B, H, Nk, d), 1.0, dtype, seed, name, "v", device)
    kl = None
    if key_lens is not None:
        kl = torch.tensor(key_lens, dtype=torch.int32, device=device)
    return {"q": q, "k": k, "v": v, "key_lens": kl}


@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    rows: int
    cols: int
    dtype: str          # "f32" or "bf16"
    sigma: float = 3.0
    masked: bool = True  # -inf beyond a per-row valid prefix (see module doc)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def describe(self) -> str:
        m = " valid prefix U{0..cols} (first full, last empty)" if self.masked else ""
        return f"row softmax rows={self.rows} cols={self.cols} {self.dtype} x~N(0,{self.sigma ** 2:g}){m}"


# Rows wider than a workgroup's on-chip share: 1024 score rows of a 256 Ki
# context in fp32 (1 GiB in, 1 GiB out).
SOFTMAX_WORKLOADS = {
    w.name: w for w in [
        SoftmaxWorkload("softmax_f32_r1024_c262144", 1024, 262144, "f32"),
    ]
}


def draw_valid_lens(rows: int, cols: int, base_seed: int, name: str) -> torch.Tensor:
    """int64 [rows]: uniform on {0..cols}; row 0 gets cols, the last row 0."""
    g = _generator(derive_seed(base_seed, name, "valid_lens", 0), "cpu")
    n = torch.randint(0, cols + 1, (rows,), generator=g, dtype=torch.int64)
    n[0] = cols
    n[rows - 1] = 0
    return n


def make_logits(rows: int, cols: int, dtype: torch.dtype, sigma: float, base_seed: int, name: str,
                masked: bool = True, device: str = "cpu", gen_device: Optional[str] = None) -> torch.Tensor:
    """[rows, cols] logits following the row-softmax recipe of the module doc."""
    gen_device = gen_device or ("cuda" if str(device).startswith("cuda") else "cpu")
    x = torch.empty((rows, cols), dtype=dtype, device=device)
    if rows == 0 or cols == 0:
        return x
    block = max(1, (1 << 22) // cols)
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        g = _generator(derive_seed(base_seed, name, "x", r0), gen_device)
        v = torch.randn((r1 - r0, cols), generator=g, device=gen_device, dtype=torch.float32)
        if sigma != 1.0:
            v.mul_(sigma)
        x[r0:r1].copy_(v.to(dtype))
    if masked:
        n = draw_valid_lens(rows, cols, base_seed, name).to(device)
        pos = torch.arange(cols, device=device)
        for r0 in range(0, rows, block):
            r1 = min(rows, r0 + block)
            x[r0:r1].masked_fill_(pos[None, :] >= n[r0:r1, None], float("-inf"))
    return x


def make_softmax_input(w: SoftmaxWorkload, base_seed: int = 0, device: str = "cpu",
                       gen_device: Optional[str] = None) -> torch.Tensor:
    return make_logits(w.rows, w.cols, w.torch_dtype, w.sigma, base_seed, w.name, w.masked,
                       device, gen_device)
