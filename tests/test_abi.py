"""The C ABI on the CPU: the library loads, exports what include/fa.h declares,
and rejects bad arguments before launching anything (no GPU is touched: every
call here returns from the host-side checks)."""
import ctypes
import os
import re
import subprocess

import pytest

import attention_forward_online_amd as fa
from attention_forward_online_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# fake, 16-byte aligned, never dereferenced: every call below fails validation
P = 0x10000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fabuild.LIB_PATH):
        fabuild.build()
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fabuild.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_testing_header_symbols_are_exported(lib):
    text = open(os.path.join(ROOT, "include", "fa_testing.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*void\s+(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)
    assert names == ["fa_testing_set_softmax_spin_limit", "fa_testing_set_rescale_rule"]
    out = subprocess.run(["nm", "-D", "--defined-only", fabuild.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert n in out
    lib.fa_testing_set_softmax_spin_limit(-1)   # host-only: no device work
    lib.fa_testing_set_rescale_rule(-1)


def test_status_strings(lib):
    assert fa.status_str(fa.FA_OK) == "FA_OK"
    assert fa.status_str(fa.FA_ERR_INVALID_ARG) == "FA_ERR_INVALID_ARG"
    assert fa.status_str(fa.FA_ERR_UNSUPPORTED) == "FA_ERR_UNSUPPORTED"
    assert fa.status_str(fa.FA_ERR_HIP) == "FA_ERR_HIP"
    assert fa.status_str(99) == "FA_ERR_UNKNOWN"
    assert lib.fa_last_hip_error() == b""


def fwd(lib, Q=P, K=P, V=P, O=P, LSE=P, B=1, H=1, N=4, Nk=4, d=64, scale=0.125, causal=0,
        key_lens=None, dtype=fa.FA_BF16):
    return lib.fa_forward(Q, K, V, O, LSE, B, H, N, Nk, d, scale, causal, key_lens, dtype, None)


def test_forward_rejects_bad_arguments(lib):
    bad = fa.FA_ERR_INVALID_ARG
    assert fwd(lib, dtype=7) == bad
    assert fwd(lib, B=-1) == bad and fwd(lib, H=-1) == bad
    assert fwd(lib, N=-1) == bad and fwd(lib, Nk=-1) == bad
    assert fwd(lib, d=0) == bad and fwd(lib, d=-64) == bad
    assert fwd(lib, causal=2) == bad
    assert fwd(lib, scale=float("nan")) == bad and fwd(lib, scale=float("inf")) == bad
    assert fwd(lib, Q=None) == bad and fwd(lib, O=None) == bad and fwd(lib, LSE=None) == bad
    assert fwd(lib, K=None) == bad and fwd(lib, V=None) == bad
    assert fwd(lib, Q=P + 2) == bad and fwd(lib, O=P + 8) == bad and fwd(lib, K=P + 4) == bad
    assert fwd(lib, LSE=P + 2) == bad
    assert fwd(lib, key_lens=P + 1) == bad
    # one (b, h) slice of 2 GiB or more
    assert fwd(lib, N=1 << 24, Nk=4, d=64) == bad
    assert fwd(lib, N=4, Nk=1 << 24, d=64, dtype=fa.FA_F32) == bad
    # grid beyond the hardware limit
    assert fwd(lib, B=65536, H=65536, N=128, d=64) == bad


def test_forward_unsupported_is_explicit(lib):
    uns = fa.FA_ERR_UNSUPPORTED
    for d in (32, 96, 80, 256):
        assert fwd(lib, d=d, dtype=fa.FA_BF16) == uns
    assert fwd(lib, d=257, dtype=fa.FA_F32) == uns
    assert fwd(lib, scale=0.0) == uns and fwd(lib, scale=-0.5) == uns


def test_forward_empty_is_a_noop(lib):
    # nothing to compute: returns before any pointer is looked at
    assert fwd(lib, Q=None, K=None, V=None, O=None, LSE=None, B=0) == fa.FA_OK
    assert fwd(lib, Q=None, K=None, V=None, O=None, LSE=None, H=0) == fa.FA_OK
    assert fwd(lib, Q=None, K=None, V=None, O=None, LSE=None, N=0) == fa.FA_OK


def test_workspace_bytes(lib):
    assert fa.fa_decode_workspace_bytes(64, 32, 128, 16) == 64 * 32 * 16 * 130 * 4
    assert fa.fa_decode_workspace_bytes(1, 1, 64, 1) == 66 * 4
    assert fa.fa_decode_workspace_bytes(-1, 1, 64, 1) == 0
    assert fa.fa_decode_workspace_bytes(1, 1, 64, 0) == 0


def dec(lib, Q=P, K=P, V=P, O=P, LSE=P, B=2, H=2, Nk=64, d=128, scale=0.1, key_lens=None,
        S=4, ws=P, ws_bytes=None, dtype=fa.FA_BF16):
    if ws_bytes is None:
        ws_bytes = lib.fa_decode_workspace_bytes(B, H, d, S)
    return lib.fa_decode_splitkv(Q, K, V, O, LSE, B, H, Nk, d, scale, key_lens, S, ws, ws_bytes,
                                 dtype, None)


def test_decode_rejects_bad_arguments(lib):
    bad, uns = fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED
    assert dec(lib, dtype=3) == bad
    assert dec(lib, S=0, ws_bytes=1 << 20) == bad
    assert dec(lib, ws=None) == bad
    assert dec(lib, ws_bytes=10) == bad
    assert dec(lib, ws_bytes=lib.fa_decode_workspace_bytes(2, 2, 128, 4) - 4) == bad
    assert dec(lib, ws=P + 4) == bad
    assert dec(lib, Q=None) == bad and dec(lib, K=None) == bad and dec(lib, LSE=None) == bad
    assert dec(lib, Nk=-1) == bad and dec(lib, d=0) == bad
    assert dec(lib, scale=float("nan")) == bad
    assert dec(lib, B=70000, ws_bytes=1 << 40) == bad
    assert dec(lib, B=1, H=1, Nk=1 << 23, ws_bytes=1 << 20) == bad
    assert dec(lib, d=96) == uns and dec(lib, d=256) == uns
    # fp32 rows of any width up to 256, as the fp32 forward
    assert dec(lib, d=257, dtype=fa.FA_F32) == uns
    assert dec(lib, S=257, ws_bytes=1 << 30) == uns
    assert dec(lib, scale=0.0) == uns
    assert dec(lib, Q=None, K=None, V=None, O=None, LSE=None, ws=None, B=0) == fa.FA_OK


def dec_na(lib, Q=P, K=P, V=P, O=P, LSE=P, B=2, H=2, Nk=64, d=128, scale=0.1, key_lens=None,
           S=4, dtype=fa.FA_BF16):
    return lib.fa_decode_splitkv_noalloc(Q, K, V, O, LSE, B, H, Nk, d, scale, key_lens, S, dtype, None)


def test_decode_noalloc_checks_before_any_launch(lib):
    # the scratch limit and every argument check answer on the host, before the
    # device is touched (no GPU here)
    limit = lib.fa_decode_scratch_bytes()
    assert limit == 32 << 20
    # the decode workload (B=64, H=32, d=128, 16 splits: 17.0 MB) fits
    assert lib.fa_decode_workspace_bytes(64, 32, 128, 16) <= limit
    # one more split per head than fits
    S = 64
    B = limit // (32 * S * (128 + 2) * 4) + 1
    assert lib.fa_decode_workspace_bytes(B, 32, 128, S) > limit
    assert dec_na(lib, B=B, H=32, S=S) == fa.FA_ERR_SCRATCH_LIMIT
    assert fa.status_str(fa.FA_ERR_SCRATCH_LIMIT) == "FA_ERR_SCRATCH_LIMIT"
    bad, uns = fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED
    assert dec_na(lib, dtype=3) == bad and dec_na(lib, S=0) == bad
    assert dec_na(lib, Q=None) == bad and dec_na(lib, K=None) == bad and dec_na(lib, LSE=None) == bad
    assert dec_na(lib, Q=P + 4) == bad and dec_na(lib, Nk=-1) == bad
    assert dec_na(lib, scale=float("nan")) == bad
    assert dec_na(lib, d=96) == uns and dec_na(lib, S=257) == uns and dec_na(lib, scale=0.0) == uns
    assert dec_na(lib, Q=None, K=None, V=None, O=None, LSE=None, B=0) == fa.FA_OK


def wsz(rows, chunks):
    return 16 + rows * chunks * 8


def test_softmax_workspace_bytes(lib):
    f32, bf = fa.FA_F32, fa.FA_BF16
    # rows that fit one workgroup's chunk need no workspace
    assert lib.fa_softmax_workspace_bytes(100, 1, f32) == 0
    assert lib.fa_softmax_workspace_bytes(100, 8192, f32) == 0
    assert lib.fa_softmax_workspace_bytes(100, 8192, bf) == 0
    assert lib.fa_softmax_workspace_bytes(100, 8185, bf) == 0
    assert lib.fa_softmax_workspace_bytes(100, 8186, bf) == wsz(100, 2)
    assert lib.fa_softmax_workspace_bytes(5, 0, f32) == 0
    # wider rows: a 16-byte header (a counter), then one 8-byte (m, l) pair per
    # (row, 8192-element chunk); a row that does not start on a 16-byte
    # boundary may need one more chunk
    assert lib.fa_softmax_workspace_bytes(1024, 262144, f32) == wsz(1024, 32)
    assert lib.fa_softmax_workspace_bytes(7, 8193, f32) == wsz(7, 2)
    assert lib.fa_softmax_workspace_bytes(3, 16381, f32) == wsz(3, 2)
    assert lib.fa_softmax_workspace_bytes(3, 16384, f32) == wsz(3, 2)
    assert lib.fa_softmax_workspace_bytes(3, 16385, f32) == wsz(3, 3)
    assert lib.fa_softmax_workspace_bytes(2, 16385, bf) == wsz(2, 3)
    assert lib.fa_softmax_workspace_bytes(2, 16384, bf) == wsz(2, 2)
    assert lib.fa_softmax_workspace_bytes(-1, 10, f32) == 0
    assert lib.fa_softmax_workspace_bytes(1, -1, f32) == 0
    assert lib.fa_softmax_workspace_bytes(1, 10, 7) == 0


def smx(lib, X=P, Y=P, LSE=P, rows=4, cols=100000, dtype=fa.FA_F32, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_softmax_workspace_bytes(rows, cols, dtype)
    return lib.fa_softmax(X, Y, LSE, rows, cols, dtype, ws, ws_bytes, None)


def test_softmax_rejects_bad_arguments(lib):
    bad = fa.FA_ERR_INVALID_ARG
    assert smx(lib, dtype=2) == bad
    assert smx(lib, rows=-1) == bad and smx(lib, cols=-1) == bad
    assert smx(lib, LSE=None) == bad and smx(lib, LSE=P + 2) == bad
    assert smx(lib, X=None) == bad and smx(lib, X=P + 4) == bad
    assert smx(lib, Y=P + 8) == bad
    assert smx(lib, ws=None) == bad and smx(lib, ws=P + 8) == bad
    assert smx(lib, ws_bytes=lib.fa_softmax_workspace_bytes(4, 100000, fa.FA_F32) - 8) == bad
    assert smx(lib, cols=(1 << 30) + 1, ws_bytes=1 << 40) == bad
    assert smx(lib, rows=1 << 20, cols=1 << 27, ws_bytes=1 << 40) == bad
    # nothing to do: no launch, no pointer is looked at
    assert smx(lib, X=None, Y=None, LSE=None, ws=None, rows=0) == fa.FA_OK


def test_backward_workspace_and_arguments(lib):
    assert lib.fa_backward_workspace_bytes(4, 16, 2048) == 8 * 4 * 16 * 2048
    assert lib.fa_backward_workspace_bytes(1, 2, 77) == 8 * 2 * 128
    assert lib.fa_backward_workspace_bytes(1, 1, 0) == 0
    assert lib.fa_backward_workspace_bytes(-1, 1, 5) == 0

    def bwd(Q=P, K=P, V=P, O=P, dO=P, LSE=P, dQ=P, dK=P, dV=P, B=1, H=2, N=100, Nk=100, d=64,
            scale=0.125, causal=0, key_lens=None, ws=P, ws_bytes=None, dtype=fa.FA_BF16):
        if ws_bytes is None:
            ws_bytes = lib.fa_backward_workspace_bytes(B, H, N)
        return lib.fa_backward(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, N, Nk, d, scale, causal,
                               key_lens, ws, ws_bytes, dtype, None)
    bad, uns = fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED
    assert bwd(dtype=5) == bad and bwd(B=-1) == bad and bwd(causal=2) == bad
    assert bwd(scale=float("inf")) == bad
    assert bwd(dtype=fa.FA_F32, d=257) == uns and bwd(d=96) == uns and bwd(scale=-1.0) == uns
    assert bwd(dO=None) == bad and bwd(LSE=None) == bad and bwd(dK=None) == bad
    assert bwd(dQ=P + 8) == bad and bwd(LSE=P + 2) == bad
    assert bwd(ws=None) == bad and bwd(ws_bytes=16) == bad
    assert bwd(B=0, Q=None, K=None, V=None, O=None, dO=None, LSE=None, dQ=None, dK=None,
               dV=None, ws=None) == fa.FA_OK


def test_python_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        fa.load_library(str(tmp_path / "libfa.so"))


def test_probe_header_symbols_are_exported_and_check_arguments(lib):
    # include/fa_probe.h: the measurement probes; every call here fails the
    # host-side checks, so nothing is launched
    text = open(os.path.join(ROOT, "include", "fa_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*fa_status\s+(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)
    assert names == ["fa_probe_mfma", "fa_probe_read", "fa_probe_copy"]
    out = subprocess.run(["nm", "-D", "--defined-only", fabuild.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert n in out
    bad = fa.FA_ERR_INVALID_ARG
    assert lib.fa_probe_mfma(None, 1, 1, None) == bad
    assert lib.fa_probe_mfma(P, 0, 1, None) == bad
    assert lib.fa_probe_mfma(P, 1, 0, None) == bad
    assert lib.fa_probe_mfma(P + 2, 1, 1, None) == bad
    assert lib.fa_probe_read(None, 16, P, 1, None) == bad
    assert lib.fa_probe_read(None, 0, None, 1, None) == bad
    assert lib.fa_probe_read(P, 16, None, 1, None) == bad
    assert lib.fa_probe_read(P, 17, P, 1, None) == bad
    assert lib.fa_probe_read(P + 8, 16, P, 1, None) == bad
    assert lib.fa_probe_read(P, 16, P, 0, None) == bad
    Q = P + (1 << 20)
    assert lib.fa_probe_copy(P, Q, 16, 0, None) == bad          # no workgroup
    assert lib.fa_probe_copy(P, Q, 24, 1, None) == bad          # not a multiple of 16
    assert lib.fa_probe_copy(None, Q, 16, 1, None) == bad
    assert lib.fa_probe_copy(P, None, 16, 1, None) == bad
    assert lib.fa_probe_copy(P + 8, Q, 16, 1, None) == bad      # misaligned
    assert lib.fa_probe_copy(P, Q + 8, 16, 1, None) == bad
    assert lib.fa_probe_copy(P, P + 16, 32, 1, None) == bad     # overlapping ranges
    assert lib.fa_probe_copy(P + 16, P, 32, 1, None) == bad
    assert lib.fa_probe_copy(None, None, 0, 1, None) == fa.FA_OK   # nothing to copy, nothing launched
