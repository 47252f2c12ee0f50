"""Python binding of the C ABI in include/fa.h (argument marshalling only).

Each function passes device pointers of torch tensors, their sizes and torch's
current HIP stream to the same-named entry point of libfa.so; every step of the
computation runs in the library's kernels.  There is no fallback: if libfa.so
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
FA_F32, FA_BF16 = 0, 1

#: every symbol include/fa.h declares
EXPORTS = ("fa_forward", "fa_decode_workspace_bytes", "fa_decode_splitkv",
           "fa_decode_splitkv_noalloc", "fa_decode_scratch_bytes",
           "fa_softmax_workspace_bytes", "fa_softmax", "fa_forward_v1_workspace_bytes",
           "fa_forward_v1", "fa_backward_workspace_bytes", "fa_backward",
           "fa_status_str", "fa_last_hip_error")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        name = status_str(status) if _lib is not None else str(status)
        super().__init__(f"{where}: {name}{(' (' + detail + ')') if detail else ''}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so and declare the ABI.  Raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m attention_forward_online_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp]
    lib.fa_forward.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp, i, vp, sz, i, vp]
    lib.fa_decode_splitkv.restype = i
    lib.fa_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp, i, i, vp]
    lib.fa_decode_splitkv_noalloc.restype = i
    lib.fa_decode_scratch_bytes.argtypes = []
    lib.fa_decode_scratch_bytes.restype = sz
    i64 = ctypes.c_int64
    lib.fa_softmax_workspace_bytes.argtypes = [i64, i64, i]
    lib.fa_softmax_workspace_bytes.restype = sz
    lib.fa_softmax.argtypes = [vp, vp, vp, i64, i64, i, vp, sz, vp]
    lib.fa_softmax.restype = i
    lib.fa_forward_v1_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_forward_v1_workspace_bytes.restype = sz
    lib.fa_forward_v1.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, sz, i, vp]
    lib.fa_forward_v1.restype = i
    lib.fa_backward_workspace_bytes.argtypes = [i, i, i]
    lib.fa_backward_workspace_bytes.restype = sz
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, sz,
                                i, vp]
    lib.fa_backward.restype = i
    lib.fa_testing_set_softmax_spin_limit.argtypes = [i]
    lib.fa_testing_set_softmax_spin_limit.restype = None
    lib.fa_testing_set_rescale_rule.argtypes = [i]
    lib.fa_testing_set_rescale_rule.restype = None
    lib.fa_probe_mfma.argtypes = [vp, i, i, vp]
    lib.fa_probe_mfma.restype = i
    lib.fa_probe_read.argtypes = [vp, sz, vp, i, vp]
    lib.fa_probe_read.restype = i
    lib.fa_probe_copy.argtypes = [vp, vp, sz, i, vp]
    lib.fa_probe_copy.restype = i
    lib.fa_status_str.argtypes = [i]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# raw handle of torch's current stream on a GPU (a private but stable torch
# entry point; the public one builds a Stream object on every call)
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _check_dev(name: str, t, dtype=None, idx: Optional[int] = None) -> None:
    """`t` must be a contiguous GPU tensor, of `dtype` and on GPU `idx` when given.
    The passing case is one combined test; a message is built only on failure."""
    if (isinstance(t, torch.Tensor) and t.is_cuda and (dtype is None or t.dtype == dtype)
            and (idx is None or t.get_device() == idx) and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if idx is not None and t.get_device() != idx:
        raise ValueError(f"{name} is on cuda:{t.get_device()}, the other tensors on cuda:{idx}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    raise ValueError(f"{name} must be contiguous")


def _launch(idx: int, stream, call):
    """Run call(stream handle) with GPU `idx` current.  `stream` (default: torch's
    current stream of that GPU) must belong to it."""
    if stream is not None and stream.device_index != idx:
        raise ValueError(f"stream is on cuda:{stream.device_index}, the tensors on cuda:{idx}")

    def handle():
        if stream is not None:
            return stream.cuda_stream
        if _raw_current_stream is not None:
            return _raw_current_stream(idx)
        return torch.cuda.current_stream(idx).cuda_stream

    if torch.cuda.current_device() == idx:
        return call(handle())
    with torch.cuda.device(idx):
        return call(handle())


def _forward_args(q, k, v, o, lse, scale, causal, key_lens):
    """Checked arguments of fa_forward (all but the stream) and the GPU index."""
    _check_dev("q", q)
    idx = q.get_device()
    for n, t in (("k", k), ("v", v), ("o", o)):
        _check_dev(n, t, q.dtype, idx)
    _check_dev("lse", lse, torch.float32, idx)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != (B, H, Nk, d) or o.shape != q.shape \
            or lse.shape != (B, H, N):
        raise ValueError("shape mismatch between q, k, v, o and lse")
    if key_lens is not None:
        _check_dev("key_lens", key_lens, torch.int32, idx)
        if key_lens.shape != (B,):
            raise ValueError("key_lens must have shape [B]")
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    return idx, (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, Nk, d, float(scale),
                 int(bool(causal)), _ptr(key_lens), _dtype_code(q))


def _raise_on(st: int, where: str, lib) -> None:
    if st != FA_OK:
        raise FaError(st, where, lib.fa_last_hip_error().decode() if st == FA_ERR_HIP else "")


def fa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
               lse: torch.Tensor, scale: Optional[float] = None, causal: bool = False,
               key_lens: Optional[torch.Tensor] = None, stream=None) -> None:
    """O, LSE <- attention(q, k, v) through the C entry point fa_forward.

    q, o: [B,H,N,d]; k, v: [B,H,Nk,d]; lse: float32 [B,H,N]; key_lens: int32 [B] or None.
    """
    lib = _lib or load_library()
    idx, args = _forward_args(q, k, v, o, lse, scale, causal, key_lens)
    _raise_on(_launch(idx, stream, lambda h: lib.fa_forward(*args, h)), "fa_forward", lib)


def _bound(lib, fn, idx, stream, args, where, tensors):
    """A launcher of fn(*args, stream handle) with the stream resolved now; each
    call runs with the tensors' GPU current, as the checked calls do.  It holds
    references to `tensors` (those whose addresses are in args), so they live
    as long as the launcher does."""
    h = _launch(idx, stream, lambda handle: handle)

    def run() -> None:
        if torch.cuda.current_device() == idx:
            st = fn(*args, h)
        else:
            with torch.cuda.device(idx):
                st = fn(*args, h)
        if st != FA_OK:
            _raise_on(st, where, lib)
    run.tensors = tuple(tensors)
    return run


def bind_forward(q, k, v, o, lse, scale=None, causal=False, key_lens=None, stream=None):
    """Check the arguments of fa_forward once and return a callable that runs it
    again on the same buffers and stream (torch's current stream of the tensors'
    GPU when binding, unless `stream` is given) without re-checking them: for
    timed loops and serving loops whose buffers stay fixed.  The callable keeps
    the tensors alive; new inputs are copied into them in place."""
    lib = _lib or load_library()
    idx, args = _forward_args(q, k, v, o, lse, scale, causal, key_lens)
    return _bound(lib, lib.fa_forward, idx, stream, args, "fa_forward", (q, k, v, o, lse, key_lens))


def fa_decode_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(load_library().fa_decode_workspace_bytes(B, H, d, num_splits))


def _decode_shapes(q, k, v, o, lse, key_lens, idx):
    for n, t in (("k", k), ("v", v), ("o", o)):
        _check_dev(n, t, q.dtype, idx)
    _check_dev("lse", lse, torch.float32, idx)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if N != 1 or k.shape != (B, H, Nk, d) or v.shape != (B, H, Nk, d) or o.shape != q.shape \
            or lse.shape != (B, H, 1):
        raise ValueError("decode expects q, o [B,H,1,d], k, v [B,H,Nk,d], lse [B,H,1]")
    if key_lens is not None:
        _check_dev("key_lens", key_lens, torch.int32, idx)
        if key_lens.shape != (B,):
            raise ValueError("key_lens must have shape [B]")
    return B, H, Nk, d


def fa_decode_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                      lse: torch.Tensor, num_splits: int, workspace: torch.Tensor,
                      scale: Optional[float] = None, key_lens: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """One-query split-KV decode through the C entry point fa_decode_splitkv.

    q, o: [B,H,1,d]; k, v: [B,H,Nk,d]; lse: float32 [B,H,1]; workspace: a GPU
    tensor of at least fa_decode_workspace_bytes(B, H, d, num_splits) bytes.
    """
    lib = _lib or load_library()
    _check_dev("q", q)
    idx = q.get_device()
    B, H, Nk, d = _decode_shapes(q, k, v, o, lse, key_lens, idx)
    _check_dev("workspace", workspace, None, idx)
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _launch(idx, stream, lambda h: lib.fa_decode_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nk, d, float(scale),
        _ptr(key_lens), int(num_splits), _ptr(workspace), ws_bytes, _dtype_code(q), h))
    if st != FA_OK:
        raise FaError(st, "fa_decode_splitkv",
                      lib.fa_last_hip_error().decode() if st == FA_ERR_HIP else "")


def fa_decode_scratch_bytes() -> int:
    return int(load_library().fa_decode_scratch_bytes())


def fa_decode_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                              lse: torch.Tensor, num_splits: int, scale: Optional[float] = None,
                              key_lens: Optional[torch.Tensor] = None, stream=None) -> None:
    """The same decode through fa_decode_splitkv_noalloc: no workspace argument,
    the partials go to the library's fixed per-GPU scratch (nothing is
    allocated).  Calls that overlap in time on one GPU race."""
    lib = _lib or load_library()
    _check_dev("q", q)
    idx = q.get_device()
    B, H, Nk, d = _decode_shapes(q, k, v, o, lse, key_lens, idx)
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    st = _launch(idx, stream, lambda h: lib.fa_decode_splitkv_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nk, d, float(scale),
        _ptr(key_lens), int(num_splits), _dtype_code(q), h))
    if st != FA_OK:
        raise FaError(st, "fa_decode_splitkv_noalloc",
                      lib.fa_last_hip_error().decode() if st == FA_ERR_HIP else "")


def fa_softmax_workspace_bytes(rows: int, cols: int, dtype: torch.dtype) -> int:
    code = FA_BF16 if dtype == torch.bfloat16 else FA_F32
    return int(load_library().fa_softmax_workspace_bytes(int(rows), int(cols), code))


def fa_softmax(x: torch.Tensor, y: Optional[torch.Tensor], lse: torch.Tensor,
               workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Row softmax and log-sum-exp through the C entry point fa_softmax.

    x: [rows, cols] float32 or bfloat16; y: same shape and dtype (may be x
    itself), or None for log-sum-exp only; lse: float32 [rows]; workspace: a
    GPU tensor of at least fa_softmax_workspace_bytes(rows, cols, dtype) bytes
    (None when that is 0).
    """
    lib = _lib or load_library()
    _check_dev("x", x)
    idx = x.get_device()
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    rows, cols = x.shape
    if y is not None:
        _check_dev("y", y, x.dtype, idx)
        if y.shape != x.shape:
            raise ValueError("y must have the shape of x")
    _check_dev("lse", lse, torch.float32, idx)
    if lse.shape != (rows,):
        raise ValueError("lse must have shape [rows]")
    ws_bytes = 0
    if workspace is not None:
        _check_dev("workspace", workspace, None, idx)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = _launch(idx, stream, lambda h: lib.fa_softmax(
        _ptr(x), _ptr(y), _ptr(lse), rows, cols, _dtype_code(x), _ptr(workspace), ws_bytes, h))
    if st != FA_OK:
        raise FaError(st, "fa_softmax", lib.fa_last_hip_error().decode() if st == FA_ERR_HIP else "")


def fa_forward_v1_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_forward_v1_workspace_bytes(B, H, N, d))


def fa_forward_v1(q, k, v, o, lse, workspace, scale=None, causal=False, key_lens=None,
                  stream=None) -> None:
    """The forward in the V1 loop order (ablation) through fa_forward_v1."""
    lib = _lib or load_library()
    _check_dev("q", q)
    idx = q.get_device()
    for n, t in (("k", k), ("v", v), ("o", o)):
        _check_dev(n, t, q.dtype, idx)
    _check_dev("lse", lse, torch.float32, idx)
    _check_dev("workspace", workspace, None, idx)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or o.shape != q.shape or lse.shape != (B, H, N):
        raise ValueError("shape mismatch between q, k, v, o and lse")
    if key_lens is not None:
        _check_dev("key_lens", key_lens, torch.int32, idx)
        if key_lens.shape != (B,):
            raise ValueError("key_lens must have shape [B]")
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _launch(idx, stream, lambda h: lib.fa_forward_v1(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, Nk, d, float(scale),
        int(bool(causal)), _ptr(key_lens), _ptr(workspace), ws_bytes, _dtype_code(q), h))
    if st != FA_OK:
        raise FaError(st, "fa_forward_v1", lib.fa_last_hip_error().decode() if st == FA_ERR_HIP else "")


def attention_v1(q, k, v, scale=None, causal=False, key_lens=None):
    """Allocate O, LSE and the workspace, run fa_forward_v1, return (O, LSE)."""
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    nbytes = fa_forward_v1_workspace_bytes(B, H, N, d)
    ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=q.device)
    fa_forward_v1(q, k, v, o, lse, ws, scale=scale, causal=causal, key_lens=key_lens)
    return o, lse


def fa_backward_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load_library().fa_backward_workspace_bytes(B, H, N))


def _backward_args(q, k, v, o, do, lse, dq, dk, dv, workspace, scale, causal, key_lens):
    """Checked arguments of fa_backward (all but the stream) and the GPU index."""
    _check_dev("q", q)
    idx = q.get_device()
    for n, t in (("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_dev(n, t, q.dtype, idx)
    _check_dev("lse", lse, torch.float32, idx)
    _check_dev("workspace", workspace, None, idx)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if (k.shape != (B, H, Nk, d) or v.shape != k.shape or dk.shape != k.shape or dv.shape != k.shape
            or o.shape != q.shape or do.shape != q.shape or dq.shape != q.shape
            or lse.shape != (B, H, N)):
        raise ValueError("shape mismatch between q, k, v, o, do, lse and the gradients")
    if key_lens is not None:
        _check_dev("key_lens", key_lens, torch.int32, idx)
        if key_lens.shape != (B,):
            raise ValueError("key_lens must have shape [B]")
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    ws_bytes = workspace.numel() * workspace.element_size()
    return idx, (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                 _ptr(dv), B, H, N, Nk, d, float(scale), int(bool(causal)), _ptr(key_lens),
                 _ptr(workspace), ws_bytes, _dtype_code(q))


def fa_backward(q, k, v, o, do, lse, dq, dk, dv, workspace, scale=None, causal=False,
                key_lens=None, stream=None) -> None:
    """dQ, dK, dV of sum(dO * O) through the C entry point fa_backward.

    q, o, do, dq: [B,H,N,d]; k, v, dk, dv: [B,H,Nk,d] (bf16); lse: float32
    [B,H,N] from fa_forward; workspace: a GPU tensor of at least
    fa_backward_workspace_bytes(B, H, N) bytes.
    """
    lib = _lib or load_library()
    idx, args = _backward_args(q, k, v, o, do, lse, dq, dk, dv, workspace, scale, causal, key_lens)
    _raise_on(_launch(idx, stream, lambda h: lib.fa_backward(*args, h)), "fa_backward", lib)


def bind_backward(q, k, v, o, do, lse, dq, dk, dv, workspace, scale=None, causal=False,
                  key_lens=None, stream=None):
    """fa_backward's arguments checked once; the returned callable runs it again on
    the same buffers and stream without re-checking (see bind_forward)."""
    lib = _lib or load_library()
    idx, args = _backward_args(q, k, v, o, do, lse, dq, dk, dv, workspace, scale, causal, key_lens)
    return _bound(lib, lib.fa_backward, idx, stream, args, "fa_backward",
                  (q, k, v, o, do, lse, dq, dk, dv, workspace, key_lens))


def attention_backward(q, k, v, o, lse, do, scale=None, causal=False, key_lens=None):
    """Allocate the gradients and the workspace, run fa_backward, return (dQ, dK, dV)."""
    B, H, N, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = fa_backward_workspace_bytes(B, H, N)
    ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=q.device)
    fa_backward(q, k, v, o, do, lse, dq, dk, dv, ws, scale=scale, causal=causal, key_lens=key_lens)
    return dq, dk, dv


def testing_set_softmax_spin_limit(limit: int) -> None:
    """Test hook (include/fa_testing.h): polls of the one-pass softmax wait
    before its fallback; 0 forces the fallback, a negative value restores the
    default."""
    load_library().fa_testing_set_softmax_spin_limit(int(limit))


RESCALE_EAGER, RESCALE_THRESHOLD, RESCALE_GUARD = 0, 1, 2


def testing_set_rescale_rule(rule: int) -> None:
    """Test and ablation hook (include/fa_testing.h): how the bf16 prefill moves
    its reference max -- RESCALE_GUARD (default), RESCALE_THRESHOLD (tau = 8)
    or RESCALE_EAGER (every tile)."""
    load_library().fa_testing_set_rescale_rule(int(rule))


PROBE_THREADS = 256                  # threads per probe workgroup (include/fa_probe.h)
PROBE_MFMA_FLOPS = 4 * 8 * 32768     # bf16 FLOPs per probe-MFMA workgroup and iteration


def probe_mfma(blocks: int, iters: int, sink: Optional[torch.Tensor] = None, device=None, stream=None):
    """Measurement probe (include/fa_probe.h): `blocks` workgroups stream
    `iters` rounds of eight bf16 MFMAs (four chains) per wave.  Executed FLOPs =
    blocks * iters * PROBE_MFMA_FLOPS.  Returns the fp32 sink (one sum per
    thread)."""
    lib = _lib or load_library()
    if sink is None:
        sink = torch.empty(blocks * PROBE_THREADS, dtype=torch.float32,
                           device=device if device is not None else "cuda")
    _check_dev("sink", sink, torch.float32)
    if sink.numel() < blocks * PROBE_THREADS:
        raise ValueError("sink holds fewer than 256 * blocks values")
    idx = sink.get_device()
    st = _launch(idx, stream, lambda h: lib.fa_probe_mfma(_ptr(sink), int(blocks), int(iters), h))
    if st != FA_OK:
        raise FaError(st, "fa_probe_mfma", lib.fa_last_hip_error().decode() if st == FA_ERR_HIP else "")
    return sink


def probe_read(src: torch.Tensor, blocks: int = 2048, sink: Optional[torch.Tensor] = None, stream=None):
    """Measurement probe (include/fa_probe.h): read all bytes of `src` once with
    16-byte loads from `blocks` workgroups.  Returns the int32 sink whose XOR
    over all entries is the XOR of the buffer's 32-bit words."""
    lib = _lib or load_library()
    _check_dev("src", src)
    idx = src.get_device()
    if sink is None:
        sink = torch.empty(blocks * PROBE_THREADS, dtype=torch.int32, device=src.device)
    _check_dev("sink", sink, torch.int32, idx)
    if sink.numel() < blocks * PROBE_THREADS:
        raise ValueError("sink holds fewer than 256 * blocks values")
    nbytes = src.numel() * src.element_size()
    st = _launch(idx, stream, lambda h: lib.fa_probe_read(_ptr(src), nbytes, _ptr(sink), int(blocks), h))
    if st != FA_OK:
        raise FaError(st, "fa_probe_read", lib.fa_last_hip_error().decode() if st == FA_ERR_HIP else "")
    return sink


def probe_copy(src: torch.Tensor, dst: torch.Tensor, blocks: int = 2048, stream=None) -> torch.Tensor:
    """Measurement probe (include/fa_probe.h): copy all bytes of `src` into
    `dst` (same device, same byte size, no overlap) with 16-byte loads and
    stores from `blocks` workgroups.  Returns dst."""
    lib = _lib or load_library()
    _check_dev("src", src)
    idx = src.get_device()
    _check_dev("dst", dst, None, idx)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst must hold as many bytes as src")
    st = _launch(idx, stream, lambda h: lib.fa_probe_copy(_ptr(src), _ptr(dst), nbytes, int(blocks), h))
    if st != FA_OK:
        raise FaError(st, "fa_probe_copy", lib.fa_last_hip_error().decode() if st == FA_ERR_HIP else "")
    return dst


def softmax(x, lse_only=False, out=None):
    """Allocate what is needed, run fa_softmax, return (Y or None, LSE)."""
    rows, cols = x.shape
    y = None if lse_only else (out if out is not None else torch.empty_like(x))
    lse = torch.empty((rows,), dtype=torch.float32, device=x.device)
    nbytes = fa_softmax_workspace_bytes(rows, cols, x.dtype)
    ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=x.device) if nbytes else None
    fa_softmax(x, y, lse, ws)
    return y, lse


def attention(q, k, v, scale=None, causal=False, key_lens=None):
    """Allocate O and LSE, run fa_forward, return (O, LSE)."""
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_forward(q, k, v, o, lse, scale=scale, causal=causal, key_lens=key_lens)
    return o, lse


def decode(q, k, v, num_splits=16, scale=None, key_lens=None):
    """Allocate O, LSE and the workspace, run fa_decode_splitkv, return (O, LSE)."""
    B, H, _, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
    nbytes = fa_decode_workspace_bytes(B, H, d, num_splits)
    ws = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    fa_decode_splitkv(q, k, v, o, lse, num_splits, ws, scale=scale, key_lens=key_lens)
    return o, lse
