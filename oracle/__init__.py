"""fp64 CPU reference for the attention forward pass (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the HIP library and its Python binding never import it.  It wraps the
plain C implementation in ``oracle.c`` (three-pass safe softmax attention in
fp64, see that file's header for the definition and the readings it takes).

Inputs are numpy arrays or CPU torch tensors holding the exact stored values:
float64, float32, or bfloat16 (passed as its raw 16-bit pattern).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_DTYPE_F64, _DTYPE_F32, _DTYPE_BF16 = 0, 1, 2


def build(out_path: str = _LIB_PATH, src_path: str = _SRC, extra_flags=()) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-fPIC", "-shared", "-pthread", *extra_flags, src_path, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def load(path: str = _LIB_PATH, rebuild_if_missing: bool = True):
    """Load (building first if needed) an oracle library and declare its ABI."""
    if not os.path.exists(path):
        if not rebuild_if_missing:
            raise FileNotFoundError(path)
        build(path)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_softmax_f64.argtypes = [dp, ctypes.c_long, dp, dp, dp]
    lib.oracle_softmax_f64.restype = ctypes.c_int
    lib.oracle_attention_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p,
        dp, dp, ctypes.c_int]
    lib.oracle_attention_f64.restype = ctypes.c_int
    lib.oracle_softmax_rows_f64.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_long,
                                            ctypes.c_long, ctypes.c_void_p, dp]
    lib.oracle_softmax_rows_f64.restype = ctypes.c_int
    lib.oracle_attention_backward_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p,
        dp, dp, dp, ctypes.c_int]
    lib.oracle_attention_backward_f64.restype = ctypes.c_int
    return lib


def _get():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def _host_array(x):
    """(contiguous numpy array, dtype code) holding the exact stored values."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                raise ValueError("oracle inputs must be host tensors")
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16)), _DTYPE_BF16
            x = x.contiguous().numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, _DTYPE_F64
    if x.dtype == np.float32:
        return x, _DTYPE_F32
    if x.dtype == np.uint16:
        return x, _DTYPE_BF16
    raise TypeError(f"unsupported oracle dtype {x.dtype}")


def softmax(x, lib=None):
    """Three-pass safe softmax of a 1-D fp64 vector; -inf entries are masked.

    Returns (y, m, l) with m = max and l = sum exp(x - m); (0, -inf, 0) when all
    entries are masked.
    """
    lib = lib or _get()
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    m = ctypes.c_double()
    l = ctypes.c_double()
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_softmax_f64(x.ctypes.data_as(dp), x.size, y.ctypes.data_as(dp),
                                ctypes.byref(m), ctypes.byref(l))
    if rc != 0:
        raise RuntimeError(f"oracle_softmax_f64 returned {rc}")
    return y, m.value, l.value


def attention(q, k, v, scale=None, causal=False, key_lens=None, rows=None, nthreads=None, lib=None):
    """fp64 attention forward.

    q: [B,H,N,d]; k, v: [B,H,Nk,d] (same dtype); key_lens: int sequence [B] or
    None; rows: flat indices (b*H + h)*N + i to compute (None = all).
    Returns (O, LSE) as float64 arrays, shaped [B,H,N,d] / [B,H,N] when rows is
    None, else [len(rows), d] / [len(rows)].
    """
    lib = lib or _get()
    qa, dt = _host_array(q)
    ka, dtk = _host_array(k)
    va, dtv = _host_array(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k and v must share one dtype")
    B, H, N, d = qa.shape
    Nk = ka.shape[2]
    if ka.shape != (B, H, Nk, d) or va.shape != (B, H, Nk, d):
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kl = None
    if key_lens is not None:
        kl = np.ascontiguousarray(np.asarray(
            key_lens.cpu().numpy() if hasattr(key_lens, "cpu") else key_lens, dtype=np.int32))
        if kl.shape != (B,):
            raise ValueError("key_lens must have shape [B]")
    if rows is None:
        nrows, ridx = B * H * N, None
    else:
        ridx = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = ridx.size
    O = np.zeros((nrows, d), dtype=np.float64)
    LSE = np.zeros((nrows,), dtype=np.float64)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_attention_f64(
        qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt, B, H, N, Nk, d, float(scale),
        int(bool(causal)), kl.ctypes.data if kl is not None else None, nrows,
        ridx.ctypes.data if ridx is not None else None,
        O.ctypes.data_as(dp), LSE.ctypes.data_as(dp), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_f64 returned {rc}")
    if rows is None:
        return O.reshape(B, H, N, d), LSE.reshape(B, H, N)
    return O, LSE


def softmax_rows(x, want_y=True, lib=None):
    """Row-wise three-pass softmax of a [rows, cols] matrix (-inf entries masked).

    Returns (Y or None, LSE) as float64 arrays; LSE = -inf for a fully masked row.
    """
    lib = lib or _get()
    xa, dt = _host_array(x)
    if xa.ndim != 2:
        raise ValueError("x must be [rows, cols]")
    rows, cols = xa.shape
    Y = np.zeros((rows, cols), dtype=np.float64) if want_y else None
    LSE = np.zeros((rows,), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_softmax_rows_f64(xa.ctypes.data if xa.size else None, dt, rows, cols,
                                     Y.ctypes.data if Y is not None else None,
                                     LSE.ctypes.data_as(dp))
    if rc != 0:
        raise RuntimeError(f"oracle_softmax_rows_f64 returned {rc}")
    return Y, LSE


def attention_backward(q, k, v, do, scale=None, causal=False, key_lens=None, heads=None,
                       nthreads=None, lib=None):
    """fp64 gradients (dQ, dK, dV) of L = sum(dO * O) for O = attention(q, k, v).

    q, do: [B,H,N,d]; k, v: [B,H,Nk,d] (one dtype); heads: flat b*H + h
    indices to compute (None = all).  Returns float64 arrays shaped like the
    inputs when heads is None, else [len(heads), N|Nk, d].
    """
    lib = lib or _get()
    qa, dt = _host_array(q)
    ka, dtk = _host_array(k)
    va, dtv = _host_array(v)
    da, dtd = _host_array(do)
    if not (dt == dtk == dtv == dtd):
        raise TypeError("q, k, v and do must share one dtype")
    B, H, N, d = qa.shape
    Nk = ka.shape[2]
    if ka.shape != (B, H, Nk, d) or va.shape != (B, H, Nk, d) or da.shape != qa.shape:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kl = None
    if key_lens is not None:
        kl = np.ascontiguousarray(np.asarray(
            key_lens.cpu().numpy() if hasattr(key_lens, "cpu") else key_lens, dtype=np.int32))
        if kl.shape != (B,):
            raise ValueError("key_lens must have shape [B]")
    if heads is None:
        nh, hidx = B * H, None
    else:
        hidx = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
        nh = hidx.size
    dQ = np.zeros((nh, N, d))
    dK = np.zeros((nh, Nk, d))
    dV = np.zeros((nh, Nk, d))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_attention_backward_f64(
        qa.ctypes.data, ka.ctypes.data, va.ctypes.data, da.ctypes.data, dt, B, H, N, Nk, d,
        float(scale), int(bool(causal)), kl.ctypes.data if kl is not None else None, nh,
        hidx.ctypes.data if hidx is not None else None,
        dQ.ctypes.data_as(dp), dK.ctypes.data_as(dp), dV.ctypes.data_as(dp), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_backward_f64 returned {rc}")
    if heads is None:
        return dQ.reshape(B, H, N, d), dK.reshape(B, H, Nk, d), dV.reshape(B, H, Nk, d)
    return dQ, dK, dV
