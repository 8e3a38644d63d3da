"""ctypes binding and build step for ``cp_oracle.c`` (plain C + OpenMP).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cp_oracle.c")
_LIB = os.path.join(_HERE, "libcporacle.so")
_lib = None


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``cp_oracle.c`` (or a copy of it) with gcc into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def bind(path: str):
    """Load a compiled copy of ``cp_oracle.c`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    lib.cp_oracle_attention.restype = ctypes.c_int
    lib.cp_oracle_attention.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.cp_oracle_attention_bwd.restype = ctypes.c_int
    lib.cp_oracle_attention_bwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.cp_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = bind(_LIB)
    return _lib


def max_threads() -> int:
    return int(_load().cp_oracle_max_threads())


def attention_rows(q, k, v, rows=None, causal: bool = True, q_offset: int = 0,
                   k_offset: int = 0, n_threads: int | None = None, lib=None):
    """Float64 attention for the query rows ``rows`` (all rows if None).

    q, k, v: CPU torch tensors [S, H, D] of float32 or bfloat16 (read as
    raw bytes, widened exactly).  Returns numpy ``out [n_rows, Hq, D]`` and
    ``lse [Hq, n_rows]``.
    """
    import torch
    assert q.dtype == k.dtype == v.dtype and q.dtype in (torch.float32, torch.bfloat16)
    q, k, v = (t.detach().cpu().contiguous() for t in (q, k, v))
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    dtype = 0 if q.dtype == torch.float32 else 1
    if rows is None:
        rows_arr = None
        n_rows = Sq
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n_rows = rows_arr.size
    out = np.empty((n_rows, Hq, D), dtype=np.float64)
    lse = np.empty((Hq, n_rows), dtype=np.float64)
    if n_threads is None:
        n_threads = len(os.sched_getaffinity(0))
    rc = (lib or _load()).cp_oracle_attention(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), dtype, Sq, Sk, Hq, Hkv, D,
        q_offset, k_offset, int(bool(causal)),
        None if rows_arr is None else rows_arr.ctypes.data, n_rows,
        out.ctypes.data, lse.ctypes.data, int(n_threads))
    if rc != 0:
        raise ValueError(f"cp_oracle_attention failed with code {rc}")
    return out, lse


def attention_bwd_rows(q, k, v, dout, q_rows=(), k_rows=(), causal: bool = True,
                       q_offset: int = 0, k_offset: int = 0, n_threads: int | None = None,
                       lib=None):
    """Float64 gradients of sum(dout * out) for selected rows.

    q, k, v, dout: CPU torch tensors (q and dout [Sq, Hq, D], k and v
    [Sk, Hkv, D]) of one dtype, float32 or bfloat16.  Returns numpy
    ``dq [len(q_rows), Hq, D]``, ``dk`` and ``dv [len(k_rows), Hkv, D]``.
    """
    import torch
    ts = (q, k, v, dout)
    assert all(t.dtype == q.dtype for t in ts) and q.dtype in (torch.float32, torch.bfloat16)
    q, k, v, dout = (t.detach().cpu().contiguous() for t in ts)
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    dtype = 0 if q.dtype == torch.float32 else 1
    qr = np.ascontiguousarray(np.asarray(q_rows, dtype=np.int64))
    kr = np.ascontiguousarray(np.asarray(k_rows, dtype=np.int64))
    dq = np.zeros((qr.size, Hq, D), dtype=np.float64)
    dk = np.zeros((kr.size, Hkv, D), dtype=np.float64)
    dv = np.zeros((kr.size, Hkv, D), dtype=np.float64)
    if n_threads is None:
        n_threads = len(os.sched_getaffinity(0))
    rc = (lib or _load()).cp_oracle_attention_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dtype, Sq, Sk, Hq, Hkv, D,
        q_offset, k_offset, int(bool(causal)),
        qr.ctypes.data if qr.size else None, qr.size,
        kr.ctypes.data if kr.size else None, kr.size,
        dq.ctypes.data if qr.size else None, dk.ctypes.data if kr.size else None,
        dv.ctypes.data if kr.size else None, int(n_threads))
    if rc != 0:
        raise ValueError(f"cp_oracle_attention_bwd failed with code {rc}")
    return dq, dk, dv
