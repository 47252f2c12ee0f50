"""GPU parity of the streaming row softmax / log-sum-exp (fa_softmax) against
the fp64 oracle on the same stored inputs.

Tolerances (derived from fp32 arithmetic on exact stored inputs):
  y, fp32 output: |y - y_ref| <= 1e-5 * y_ref * (1 + |x - m| / 16) + 1e-37.
      The exponent argument x - m is rounded in fp32, so exp carries a relative
      error of about |x - m| * 2^-23; the sum l adds a few 1e-6.  The 1e-37 floor
      covers outputs below the smallest normal fp32.
  y, bf16 output: the same plus 2^-8 relative (round to nearest even to 8
      significant bits): 4e-3 * y_ref + the fp32 term.
  lse: |lse - lse_ref| <= 1e-5 + 2.4e-7 * |lse_ref| (the sum's relative
      error, and two fp32 roundings of m + ln l).
  Masked entries (x = -inf) give y = 0 exactly; a row with no finite entry
  gives y = 0 and lse = -inf exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_forward_online_amd as fa
import oracle
from attention_forward_online_amd import synth
from gpu_common import say, to_host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def check_rows(x_host: torch.Tensor, y_gpu, lse_gpu, what: str, dtype: torch.dtype):
    """Compare GPU rows (host copies of y, lse) with the oracle on x_host."""
    Y_ref, L_ref = oracle.softmax_rows(x_host, want_y=y_gpu is not None)
    lse = to_host(lse_gpu).double().numpy()
    assert not np.isnan(lse).any(), f"{what}: NaN in lse"
    masked_row = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(lse), masked_row), f"{what}: -inf pattern of lse differs"
    vis = ~masked_row
    el = 0.0
    if vis.any():
        err = np.abs(lse[vis] - L_ref[vis])
        tol = 1e-5 + 2.4e-7 * np.abs(L_ref[vis])
        el = float(err.max())
        assert np.all(err <= tol), f"{what}: max |dlse| = {el:.3e}"
    ey = 0.0
    if y_gpu is not None:
        y = to_host(y_gpu).double().numpy()
        x = x_host.double().numpy()
        assert not np.isnan(y).any(), f"{what}: NaN in y"
        assert np.all(y[np.isneginf(x)] == 0.0), f"{what}: masked entries not exactly 0"
        m = np.where(vis, np.max(np.where(np.isneginf(x), -np.inf, x), axis=1, initial=-np.inf), 0.0)
        fin = ~np.isneginf(x)
        z = np.abs(np.where(fin, x, 0.0) - m[:, None])
        tol = 1e-5 * Y_ref * (1.0 + z / 16.0) + 1e-37
        if dtype == torch.bfloat16:
            tol = tol + 4e-3 * Y_ref
        err = np.abs(y - Y_ref)
        bad = err > tol
        ey = float((err / np.maximum(Y_ref, 1e-300))[fin].max()) if fin.any() else 0.0
        assert not bad.any(), (f"{what}: {int(bad.sum())} entries out of tolerance, first at "
                               f"{np.argwhere(bad)[0].tolist()}: y={y[bad][0]!r} ref={Y_ref[bad][0]!r}")
    return ey, el


def run(x_dev, lse_only=False, out=None):
    y, lse = fa.softmax(x_dev, lse_only=lse_only, out=out)
    torch.cuda.synchronize()
    return y, lse


def case(rows, cols, dtype, sigma=3.0, seed=0, masked=True):
    name = f"smx_{rows}_{cols}_{dtype}_{sigma}"
    return synth.make_logits(rows, cols, dtype, sigma, seed, name, masked, device=DEV)


# widths around every path boundary: a wave per row (<= 2048 elements incl.
# the head offset of a row that starts off the 16-byte grid), a workgroup per
# row (<= 8192), and the two-pass path with 2, 3 and many chunks; odd widths
# make rows start off the 16-byte grid
F32_COLS = [1, 3, 4, 7, 64, 100, 2045, 2048, 2049, 5001, 8189, 8192, 8193, 16384, 16385, 40003]
BF16_COLS = [1, 5, 8, 9, 100, 2041, 2048, 2049, 5000, 8185, 8186, 8192, 8193, 16384, 16385, 50001]


@pytest.mark.parametrize("cols", F32_COLS)
def test_f32_widths(cols):
    rows = 37 if cols <= 20000 else 9
    x = case(rows, cols, torch.float32)
    say(f"[gpu] fa_softmax f32 rows={rows} cols={cols}")
    y, lse = run(x)
    check_rows(to_host(x), y, lse, f"f32 {rows}x{cols}", torch.float32)


@pytest.mark.parametrize("cols", BF16_COLS)
def test_bf16_widths(cols):
    rows = 37 if cols <= 20000 else 9
    x = case(rows, cols, torch.bfloat16)
    say(f"[gpu] fa_softmax bf16 rows={rows} cols={cols}")
    y, lse = run(x)
    check_rows(to_host(x), y, lse, f"bf16 {rows}x{cols}", torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cols", [777, 9001, 70000])
def test_scattered_masks_and_single_entry_rows(dtype, cols):
    # -inf anywhere (not only a suffix), rows with one finite entry at the
    # start, in the middle and at the end, a row of -inf only
    rows = 16
    x = case(rows, cols, dtype, masked=False)
    g = torch.Generator(device=DEV)
    g.manual_seed(1234 + cols)
    drop = torch.rand((rows, cols), generator=g, device=DEV) < 0.6
    x.masked_fill_(drop, float("-inf"))
    for r, j in ((1, 0), (2, cols // 2), (3, cols - 1)):
        x[r].fill_(float("-inf"))
        x[r, j] = 2.5
    x[4].fill_(float("-inf"))
    say(f"[gpu] fa_softmax scattered masks {dtype} cols={cols}")
    y, lse = run(x)
    check_rows(to_host(x), y, lse, f"scattered {dtype} {cols}", dtype)
    yh = to_host(y).double()
    for r, j in ((1, 0), (2, cols // 2), (3, cols - 1)):
        assert yh[r, j].item() == 1.0 and float(yh[r].sum()) == 1.0


@pytest.mark.parametrize("cols", [3000, 100000])
def test_high_dynamic_range_and_offsets(cols):
    # sigma 30 (most entries underflow against the row max) and rows shifted by
    # large offsets: softmax is shift-invariant, lse shifts by the offset
    rows = 8
    x = case(rows, cols, torch.float32, sigma=30.0)
    off = torch.tensor([0.0, 1e4, -1e4, 512.0, -3e3, 77.0, 1e5, -1e5], device=DEV)[:, None]
    x = (x + off).contiguous()
    say(f"[gpu] fa_softmax high dynamic range cols={cols}")
    y, lse = run(x)
    check_rows(to_host(x), y, lse, f"hdr {cols}", torch.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cols", [1000, 12000, 60001])
def test_lse_only_and_in_place(dtype, cols):
    rows = 11
    x = case(rows, cols, dtype)
    xh = to_host(x).clone()
    say(f"[gpu] fa_softmax lse-only / in-place {dtype} cols={cols}")
    y0, lse_only = run(x, lse_only=True)
    assert y0 is None
    # log-sum-exp only must leave x untouched
    bits = (lambda t: t.view(torch.int16)) if dtype == torch.bfloat16 else (lambda t: t)
    assert torch.equal(bits(to_host(x)), bits(xh))
    y_sep, lse_sep = run(x)
    check_rows(xh, None, lse_only, f"lse-only {dtype} {cols}", dtype)
    check_rows(xh, y_sep, lse_sep, f"separate {dtype} {cols}", dtype)
    y_in, lse_in = run(x, out=x)          # y written over x
    assert y_in.data_ptr() == x.data_ptr()
    check_rows(xh, y_in, lse_in, f"in-place {dtype} {cols}", dtype)

    # paths that cut the row into the same chunks give the same bits: rows
    # that fit one workgroup take one kernel every way; wider rows take the
    # two-pass kernels for lse only and in place (8192-element chunks) and the
    # one-pass kernel out of place (64 KiB chunks), equal to the others only
    # up to rounding
    def same(a, b, what):
        a, b = to_host(a), to_host(b)
        bad = (a != b) & ~(torch.isneginf(a) & torch.isneginf(b))
        assert not bad.any(), (f"{what}: rows {torch.nonzero(bad).flatten().tolist()} differ: "
                               f"{a[bad].tolist()} vs {b[bad].tolist()}")
    same(lse_only, lse_in, "lse-only vs in place")
    if cols + 7 <= 8192:
        same(lse_only, lse_sep, "lse-only vs separate")
        assert torch.equal(bits(to_host(y_in)), bits(to_host(y_sep)))


def test_empty_shapes():
    say("[gpu] fa_softmax empty shapes")
    x = torch.empty((5, 0), dtype=torch.float32, device=DEV)
    y, lse = run(x)
    assert y.shape == (5, 0) and torch.all(torch.isneginf(to_host(lse)))
    x = torch.empty((0, 100), dtype=torch.bfloat16, device=DEV)
    y, lse = run(x)
    assert y.shape == (0, 100) and lse.shape == (0,)


def test_deterministic_and_row_blocks():
    # 80 rows of 1 MiB.  Out of place: the one-pass path, twice, bit-identical.
    # In place: the two-pass path over more than one block of rows (64 MiB
    # each)
    rows, cols = 80, 262144
    x = case(rows, cols, torch.float32, seed=3)
    say(f"[gpu] fa_softmax one-pass / row blocks rows={rows} cols={cols}")
    y1, l1 = run(x)
    y2, l2 = run(x)
    assert torch.equal(to_host(y1), to_host(y2)) and torch.equal(to_host(l1), to_host(l2))
    xh = to_host(x)
    y3, l3 = run(x, out=x)
    pick = [0, 1, 31, 63, 64, 65, 78, 79]
    check_rows(xh[pick], to_host(y1)[pick], to_host(l1)[pick], "one-pass", torch.float32)
    check_rows(xh[pick], to_host(y3)[pick], to_host(l3)[pick], "row blocks in place", torch.float32)


@pytest.mark.parametrize("name", sorted(synth.SOFTMAX_WORKLOADS))
def test_full_size_workload(name):
    w = synth.SOFTMAX_WORKLOADS[name]
    say(f"[gpu] fa_softmax full size {w.describe()}")
    x = synth.make_softmax_input(w, device=DEV)
    y, lse = run(x)
    # sampled rows element by element against the oracle
    rng = np.random.default_rng(5)
    pick = sorted({0, 1, w.rows // 2, w.rows - 2, w.rows - 1} | set(rng.integers(0, w.rows, 6).tolist()))
    check_rows(to_host(x[pick]), to_host(y[pick]), to_host(lse[pick]), name, w.torch_dtype)
    # every row: y sums to 1 where the row has a finite entry, lse agrees with
    # a float64 log-sum-exp, masked entries are exactly 0
    fin = ~torch.isneginf(x)
    has = fin.any(dim=1)
    sums = y.double().sum(dim=1)
    assert torch.all((sums[has] - 1.0).abs() <= 1e-4)
    assert torch.all(sums[~has] == 0.0)
    ref = torch.logsumexp(x.double(), dim=1)
    d = (lse.double() - ref)[has].abs()
    assert torch.all(d <= 1e-5 + 2.4e-7 * ref[has].abs())
    assert torch.all(torch.isneginf(lse[~has]))
    assert torch.all(y[~fin] == 0)


def test_workspace_reuse_across_calls():
    # one workspace for several calls in a row (one-pass wide path, then the
    # two-pass in-place path, then one-pass again): every call resets what it
    # reads, so each result matches the oracle
    rows, cols = 6, 50000
    nbytes = fa.fa_softmax_workspace_bytes(rows, cols, torch.float32)
    ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=DEV)
    lse = torch.empty(rows, dtype=torch.float32, device=DEV)
    for k, in_place in enumerate((False, True, False, False)):
        x = case(rows, cols, torch.float32, seed=10 + k)
        xh = to_host(x).clone()
        y = x if in_place else torch.empty_like(x)
        say(f"[gpu] fa_softmax reused workspace call {k} in_place={in_place}")
        fa.fa_softmax(x, y, lse, ws)
        torch.cuda.synchronize()
        check_rows(xh, y, lse, f"reuse {k}", torch.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_one_pass_wait_fallback(dtype):
    # forced from the host: with a poll limit of 0 every workgroup of the
    # one-pass kernel computes its row's statistics by streaming the row
    # itself; the result still matches the oracle, bit for bit the waiting
    # path's
    rows, cols = 5, 70001
    x = case(rows, cols, dtype, seed=21)
    say(f"[gpu] fa_softmax one-pass fallback {dtype} rows={rows} cols={cols}")
    fa.testing_set_softmax_spin_limit(0)
    try:
        y, lse = run(x)
    finally:
        fa.testing_set_softmax_spin_limit(-1)
    check_rows(to_host(x), y, lse, f"fallback {dtype}", dtype)
    y2, lse2 = run(x)
    check_rows(to_host(x), y2, lse2, f"after fallback {dtype}", dtype)
    # the fallback forms and merges the chunk pairs exactly as the waiting path
    assert torch.equal(y, y2) and torch.equal(lse, lse2), "fallback differs from the waiting path"


# one-pass out-of-place rows hold at most 128 chunks of 64 KiB (16384 fp32 or
# 32768 bf16 elements); one element more takes the two-pass kernels
@pytest.mark.parametrize("dtype,chunk", [(torch.float32, 16384), (torch.bfloat16, 32768)])
@pytest.mark.parametrize("extra", [0, 1])
def test_rows_at_the_chunk_limit(dtype, chunk, extra):
    cols = 128 * chunk + extra
    x = case(3, cols, dtype, seed=30 + extra)
    say(f"[gpu] fa_softmax {dtype} 3 x {cols} (one-pass chunk limit {'+1' if extra else ''})")
    y, lse = run(x)
    check_rows(to_host(x), y, lse, f"{dtype} 3x{cols}", dtype)
    _, lse_only = run(x, lse_only=True)
    check_rows(to_host(x), None, lse_only, f"lse-only {dtype} 3x{cols}", dtype)


def test_widest_accepted_row():
    # the widest row the library takes (2^30 elements: its chunk indices stay
    # 32-bit), checked on the log-sum-exp; one element more is rejected
    cols = 1 << 30
    x = case(1, cols, torch.bfloat16, seed=40)
    say(f"[gpu] fa_softmax bf16 1 x {cols} (widest accepted), lse only")
    _, lse = run(x, lse_only=True)
    check_rows(to_host(x), None, lse, f"bf16 1x{cols}", torch.bfloat16)
    del x
    torch.cuda.empty_cache()
    x1 = torch.empty((1, cols + 1), dtype=torch.bfloat16, device=DEV)
    l1 = torch.empty((1,), dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError, match="FA_ERR_INVALID_ARG"):
        fa.fa_softmax(x1, None, l1)
