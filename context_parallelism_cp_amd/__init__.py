"""Python binding of libcpattn.so: blockwise causal attention with per-row
log-sum-exp, the log-sum-exp merge, the ring schedule and the Ulysses
repacks on one MI355X (gfx950).

Argument marshalling only: shapes and pointers are read from torch tensors
and handed to the C-ABI declared in ``include/cp_attn.h``; every step runs
in the library's HIP kernels on the caller's current HIP stream.  Torch
provides device memory and streams.  There is no fallback: importing this
package fails if ``libcpattn.so`` has not been built
(``python -m context_parallelism_cp_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpattn.so")

(CP_OK, CP_ERR_NULL, CP_ERR_SHAPE, CP_ERR_UNSUPPORTED, CP_ERR_CAPACITY, CP_ERR_HIP, CP_ERR_ALIGN,
 CP_ERR_WORKSPACE) = range(8)
CP_F32, CP_BF16 = 0, 1
CP_LAYOUT_CONTIGUOUS, CP_LAYOUT_ZIGZAG, CP_LAYOUT_STRIPED = 0, 1, 2
CP_PAIR_SKIP, CP_PAIR_FULL, CP_PAIR_DIAG = 0, 1, 2
(CP_KERNEL_ATTN_BF16, CP_KERNEL_ATTN_F32, CP_KERNEL_MERGE, CP_KERNEL_PERMUTE, CP_KERNEL_BWD_BF16,
 CP_KERNEL_BWD_F32, CP_KERNEL_BWD_DVEC) = range(7)

LAYOUTS = {"contiguous": CP_LAYOUT_CONTIGUOUS, "zigzag": CP_LAYOUT_ZIGZAG,
           "striped": CP_LAYOUT_STRIPED}


class CpError(RuntimeError):
    """A non-zero cp_status; ``code`` holds it."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[cp_status {code}] {msg}")
        self.code = code


class cp_block_pair(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("step", ctypes.c_int32),
                ("q_chunk", ctypes.c_int32), ("k_chunk", ctypes.c_int32),
                ("q_offset", ctypes.c_int64), ("k_offset", ctypes.c_int64),
                ("len_q", ctypes.c_int64), ("len_k", ctypes.c_int64),
                ("kind", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "cp_attn_block_fwd": [_P, _P, _P, _P, _P, _I64, _I64, _I, _I, _I, _I64, _I64, _I, _I, _P],
    "cp_lse_merge": [_P, _P, _P, _P, _P, _P, _I64, _I, _I, _P],
    "cp_ring_fwd": [_P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I, _I, _I, _P],
    "cp_attn_bwd_dvec": [_P, _P, _P, _I64, _I, _I, _I, _P],
    "cp_attn_block_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I, _I, _I, _I64,
                          _I64, _I, _I, _I, _P],
    "cp_ring_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I, _I,
                    _I, _P],
    "cp_ring_bwd_noalloc": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I,
                            _I, _I, _P],
    "cp_seq_to_head": [_P, _P, _I64, _I, _I, _I, _I, _SZ, _P],
    "cp_head_to_seq": [_P, _P, _I64, _I, _I, _I, _I, _SZ, _P],
    "cp_usp_fwd_workspace": [_I64, _I, _I, _I, _I, _I, _I, _I, _I,
                             ctypes.POINTER(ctypes.c_size_t)],
    "cp_usp_fwd": [_P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _SZ, _P],
    "cp_usp_bwd_workspace": [_I64, _I, _I, _I, _I, _I, _I, _I, _I,
                             ctypes.POINTER(ctypes.c_size_t)],
    "cp_usp_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I, _I, _I,
                   _I, _P, _SZ, _P],
    "cp_kv_seq_to_head": [_P, _P, _I64, _I, _I, _I, _I, _SZ, _P],
    "cp_layout_index": [_I, _I64, _I, _I, _P],
    "cp_ring_plan": [_I64, _I, _I, _I, _I, _P, ctypes.POINTER(ctypes.c_int)],
    "cp_last_error": [],
    "cp_timing_enable": [_I],
    "cp_timing_reset": [],
    "cp_timing_read": [_I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)],
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m context_parallelism_cp_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "cp_last_error" else ctypes.c_int
    return lib


lib = _load()


def cp_last_error() -> str:
    return lib.cp_last_error().decode()


def _check(rc: int):
    if rc != CP_OK:
        raise CpError(rc, cp_last_error())


def _stream(t, stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CP_BF16
    if t.dtype == torch.float32:
        return CP_F32
    raise CpError(CP_ERR_UNSUPPORTED, f"dtype {t.dtype} is not supported")


def _need(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise CpError(CP_ERR_SHAPE, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _checked(ref, *specs):
    """Check every tensor argument before the library is called.

    ``ref`` is the tensor whose dtype and device the others follow (q, or
    dout for cp_attn_bwd_dvec, or x for the repacks).  Each spec is
    ``(tensor, shape, kind, name)``: ``shape`` the exact shape (None: any),
    ``kind`` "in" (ref's dtype, which must be bfloat16 or float32), "f32"
    (float32), "same" (ref's dtype, any element size) or "u8" (a byte
    workspace).  Every tensor must be dense and live on ref's GPU.  The C
    side receives only pointers and sizes, so a wrong buffer would otherwise
    be read or written out of bounds by the kernels."""
    import torch
    for t, shape, kind, name in specs:
        if not torch.is_tensor(t):
            raise CpError(CP_ERR_NULL, f"{name} must be a torch tensor")
        if shape is not None:
            _need(t, shape, name)
    want = {"in": ref.dtype, "same": ref.dtype, "f32": torch.float32, "u8": torch.uint8}
    for t, shape, kind, name in specs:
        if kind == "in" and t.dtype not in (torch.bfloat16, torch.float32):
            raise CpError(CP_ERR_UNSUPPORTED, f"{name}: dtype {t.dtype} is not supported")
        if t.dtype != want[kind]:
            raise CpError(CP_ERR_UNSUPPORTED,
                          f"{name} must have dtype {want[kind]}, got {t.dtype}")
        if not t.is_contiguous():
            raise CpError(CP_ERR_ALIGN, f"{name} must be contiguous")
    if ref.device.type != "cuda":
        raise CpError(CP_ERR_UNSUPPORTED, f"tensors must live on a GPU, got {ref.device}")
    for t, shape, kind, name in specs:
        if t.device != ref.device:
            raise CpError(CP_ERR_UNSUPPORTED,
                          f"{name} must be on {ref.device} like the inputs, got {t.device}")


# ------------------------------------------------------------------ entry points
def _dims(t, n, name):
    """The sizes of a tensor that must have n dimensions."""
    import torch
    if not torch.is_tensor(t):
        raise CpError(CP_ERR_NULL, f"{name} must be a torch tensor")
    if t.dim() != n:
        raise CpError(CP_ERR_SHAPE, f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _f32(shape, ref):
    import torch
    return torch.empty(*shape, device=ref.device, dtype=torch.float32)


def cp_attn_block_fwd(q, k, v, out=None, lse=None, q_offset: int = 0, k_offset: int = 0,
                      causal: bool = True, stream=None):
    """out [Sq,Hq,D] f32 and lse [Hq,Sq] f32 of q [Sq,Hq,D] against k, v [Sk,Hkv,D]."""
    Sq, Hq, D = _dims(q, 3, "q")
    Sk, Hkv, _ = _dims(k, 3, "k")
    out = _f32((Sq, Hq, D), q) if out is None else out
    lse = _f32((Hq, Sq), q) if lse is None else lse
    _checked(q, (q, None, "in", "q"), (k, (Sk, Hkv, D), "in", "k"), (v, (Sk, Hkv, D), "in", "v"),
             (out, (Sq, Hq, D), "f32", "out"), (lse, (Hq, Sq), "f32", "lse"))
    _check(lib.cp_attn_block_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), Sq, Sk, Hq, Hkv, D, q_offset, k_offset,
                                 int(bool(causal)), _dtype_code(q), _stream(q, stream)))
    return out, lse


def cp_lse_merge(o1, lse1, o2, lse2, o=None, lse=None, stream=None):
    """Log-sum-exp merge; o may be o1 and lse may be lse1 (in place)."""
    import torch
    Sq, H, D = _dims(o1, 3, "o1")
    o = torch.empty_like(o1) if o is None else o
    lse = _f32((H, Sq), o1) if lse is None else lse
    _checked(o1, (o1, None, "f32", "o1"), (lse1, (H, Sq), "f32", "lse1"),
             (o2, (Sq, H, D), "f32", "o2"), (lse2, (H, Sq), "f32", "lse2"),
             (o, (Sq, H, D), "f32", "o"), (lse, (H, Sq), "f32", "lse"))
    _check(lib.cp_lse_merge(o1.data_ptr(), lse1.data_ptr(), o2.data_ptr(), lse2.data_ptr(),
                            o.data_ptr(), lse.data_ptr(), Sq, H, D, _stream(o1, stream)))
    return o, lse


def padded_length(S: int, P: int, layout) -> int:
    """S rounded up to a multiple of the split: P chunks, 2P for zigzag."""
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    m = 2 * P if lay == CP_LAYOUT_ZIGZAG else P
    return -(-S // max(m, 1)) * m


def _ring_rows(S: int, P: int, lay: int, rank: int):
    """(rows of q/k/v, rows of out/lse/dq) of a ring call of real length S."""
    Sp = padded_length(S, P, lay)
    rows_in = Sp if lay == CP_LAYOUT_STRIPED else S
    return rows_in, (rows_in if rank < 0 else Sp // max(P, 1))


def cp_ring_fwd(q, k, v, P: int, layout="zigzag", rank: int = -1, causal: bool = True,
                out=None, lse=None, stream=None, seq_len=None):
    """Ring attention over P virtual ranks (rank=-1: all, in the inputs'
    order -- natural, or striped for the striped layout; rank=r: that
    rank's share in its local order).  seq_len: the real length when the
    split does not divide it (striped tensors then hold the padded length;
    padding rows of the output come back as (0, -inf))."""
    _, Hq, D = _dims(q, 3, "q")
    _, Hkv, _ = _dims(k, 3, "k")
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    S = q.shape[0] if seq_len is None else int(seq_len)
    rows_in, rows = _ring_rows(S, P, lay, rank)
    out = _f32((rows, Hq, D), q) if out is None else out
    lse = _f32((Hq, rows), q) if lse is None else lse
    _checked(q, (q, (rows_in, Hq, D), "in", "q"), (k, (rows_in, Hkv, D), "in", "k"),
             (v, (rows_in, Hkv, D), "in", "v"), (out, (rows, Hq, D), "f32", "out"),
             (lse, (Hq, rows), "f32", "lse"))
    _check(lib.cp_ring_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), S, Hq, Hkv, D, P, lay, rank, int(bool(causal)),
                           _dtype_code(q), _stream(q, stream)))
    return out, lse


def cp_attn_bwd_dvec(out, dout, dvec=None, stream=None):
    """dvec[h][i] = sum_d dout[i][h][d] * out[i][h][d] (float32 [Hq][Sq])."""
    Sq, Hq, D = _dims(out, 3, "out")
    dvec = _f32((Hq, Sq), dout) if dvec is None else dvec
    _checked(dout, (dout, (Sq, Hq, D), "in", "dout"), (out, (Sq, Hq, D), "f32", "out"),
             (dvec, (Hq, Sq), "f32", "dvec"))
    _check(lib.cp_attn_bwd_dvec(out.data_ptr(), dout.data_ptr(), dvec.data_ptr(), Sq, Hq, D,
                                _dtype_code(dout), _stream(out, stream)))
    return dvec


def cp_attn_block_bwd(q, k, v, dout, lse, dvec, dq=None, dk=None, dv=None, q_offset: int = 0,
                      k_offset: int = 0, causal: bool = True, accumulate: bool = False,
                      stream=None):
    """Gradients of one query chunk against one KV block (float32 dq, dk,
    dv), from the rows' final lse and dvec; accumulate adds into dq/dk/dv."""
    Sq, Hq, D = _dims(q, 3, "q")
    Sk, Hkv, _ = _dims(k, 3, "k")
    dq = _f32((Sq, Hq, D), q) if dq is None else dq
    dk = _f32((Sk, Hkv, D), q) if dk is None else dk
    dv = _f32((Sk, Hkv, D), q) if dv is None else dv
    _checked(q, (q, None, "in", "q"), (k, (Sk, Hkv, D), "in", "k"), (v, (Sk, Hkv, D), "in", "v"),
             (dout, (Sq, Hq, D), "in", "dout"), (lse, (Hq, Sq), "f32", "lse"),
             (dvec, (Hq, Sq), "f32", "dvec"), (dq, (Sq, Hq, D), "f32", "dq"),
             (dk, (Sk, Hkv, D), "f32", "dk"), (dv, (Sk, Hkv, D), "f32", "dv"))
    _check(lib.cp_attn_block_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                 lse.data_ptr(), dvec.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                 dv.data_ptr(), Sq, Sk, Hq, Hkv, D, q_offset, k_offset,
                                 int(bool(causal)), int(bool(accumulate)), _dtype_code(q),
                                 _stream(q, stream)))
    return dq, dk, dv


def _ring_bwd_args(q, k, v, out, lse, dout, P, layout, rank, seq_len, dq, dk, dv):
    """Shapes of a ring backward call, its gradient buffers and their checks."""
    _, Hq, D = _dims(q, 3, "q")
    _, Hkv, _ = _dims(k, 3, "k")
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    S = q.shape[0] if seq_len is None else int(seq_len)
    rows_in, rows = _ring_rows(S, P, lay, rank)
    dq = _f32((rows, Hq, D), q) if dq is None else dq
    dk = _f32((rows_in, Hkv, D), q) if dk is None else dk
    dv = _f32((rows_in, Hkv, D), q) if dv is None else dv
    specs = [(q, (rows_in, Hq, D), "in", "q"), (k, (rows_in, Hkv, D), "in", "k"),
             (v, (rows_in, Hkv, D), "in", "v"), (out, (rows, Hq, D), "f32", "out"),
             (lse, (Hq, rows), "f32", "lse"), (dout, (rows, Hq, D), "in", "dout"),
             (dq, (rows, Hq, D), "f32", "dq"), (dk, (rows_in, Hkv, D), "f32", "dk"),
             (dv, (rows_in, Hkv, D), "f32", "dv")]
    return S, Hq, Hkv, D, lay, rows, dq, dk, dv, specs


def cp_ring_bwd(q, k, v, out, lse, dout, P: int, layout="zigzag", rank: int = -1,
                causal: bool = True, dq=None, dk=None, dv=None, dvec=None, stream=None,
                seq_len=None):
    """Backward of cp_ring_fwd: dq in the forward's output layout, dk and dv
    [rows of k][Hkv][D] float32 in the inputs' order -- natural, or striped
    for the striped layout (contributions of the rank(s) computed)."""
    S, Hq, Hkv, D, lay, rows, dq, dk, dv, specs = _ring_bwd_args(
        q, k, v, out, lse, dout, P, layout, rank, seq_len, dq, dk, dv)
    dvec = _f32((Hq, rows), q) if dvec is None else dvec
    _checked(q, *specs, (dvec, (Hq, rows), "f32", "dvec"))
    _check(lib.cp_ring_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                           dv.data_ptr(), dvec.data_ptr(), S, Hq, Hkv, D, P, lay, rank,
                           int(bool(causal)), _dtype_code(q), _stream(q, stream)))
    return dq, dk, dv


def cp_ring_bwd_noalloc(q, k, v, out, lse, dout, dq, dk, dv, P: int, layout="zigzag",
                        rank: int = -1, causal: bool = True, stream=None, seq_len=None):
    """cp_ring_bwd with its dvec scratch in the library's own device array:
    the library allocates nothing (dq, dk, dv are the caller's buffers).
    Calls that overlap on one GPU race (one array per GPU)."""
    S, Hq, Hkv, D, lay, rows, dq, dk, dv, specs = _ring_bwd_args(
        q, k, v, out, lse, dout, P, layout, rank, seq_len, dq, dk, dv)
    _checked(q, *specs)
    _check(lib.cp_ring_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), S, Hq, Hkv, D, P, lay, rank, int(bool(causal)),
                                   _dtype_code(q), _stream(q, stream)))
    return dq, dk, dv


def _dtype_arg(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    return CP_BF16 if str(dtype) == "torch.bfloat16" else CP_F32


def cp_usp_fwd_workspace(S: int, Hq: int, Hkv: int, D: int, P_u: int, P_r: int, layout,
                         rank: int, dtype) -> int:
    """Workspace bytes of cp_usp_fwd (dtype: CP_F32 / CP_BF16 or a torch dtype)."""
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    n = ctypes.c_size_t(0)
    _check(lib.cp_usp_fwd_workspace(S, Hq, Hkv, D, P_u, P_r, lay, rank, _dtype_arg(dtype),
                                    ctypes.byref(n)))
    return n.value


def _workspace(workspace, need, ref):
    import torch
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=ref.device, dtype=torch.uint8)
    return workspace


def cp_usp_fwd(q, k, v, P_u: int, P_r: int, layout="zigzag", rank: int = -1,
               causal: bool = True, out=None, lse=None, workspace=None, stream=None,
               seq_len=None):
    """USP hybrid on P_u * P_r virtual ranks (rank = r * P_u + u).  rank=-1:
    out, lse over the inputs' rows in their order; rank: ring group r's
    rows in its local order, head share u written.  seq_len: the real length
    when the ring split does not divide it (padded as cp_ring_fwd)."""
    _, Hq, D = _dims(q, 3, "q")
    _, Hkv, _ = _dims(k, 3, "k")
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    S = q.shape[0] if seq_len is None else int(seq_len)
    rows_in, rows = _ring_rows(S, P_r, lay, -1 if rank < 0 else rank // max(P_u, 1))
    need = cp_usp_fwd_workspace(S, Hq, Hkv, D, P_u, P_r, lay, rank, _dtype_code(q))
    out = _f32((rows, Hq, D), q) if out is None else out
    lse = _f32((Hq, rows), q) if lse is None else lse
    workspace = _workspace(workspace, need, q)
    _checked(q, (q, (rows_in, Hq, D), "in", "q"), (k, (rows_in, Hkv, D), "in", "k"),
             (v, (rows_in, Hkv, D), "in", "v"), (out, (rows, Hq, D), "f32", "out"),
             (lse, (Hq, rows), "f32", "lse"), (workspace, None, "u8", "workspace"))
    _check(lib.cp_usp_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), S, Hq, Hkv, D, P_u, P_r, lay, rank, int(bool(causal)),
                          _dtype_code(q), workspace.data_ptr(), workspace.numel(),
                          _stream(q, stream)))
    return out, lse


def cp_usp_bwd_workspace(S: int, Hq: int, Hkv: int, D: int, P_u: int, P_r: int, layout,
                         rank: int, dtype) -> int:
    """Workspace bytes of cp_usp_bwd (dtype: CP_F32 / CP_BF16 or a torch dtype)."""
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    n = ctypes.c_size_t(0)
    _check(lib.cp_usp_bwd_workspace(S, Hq, Hkv, D, P_u, P_r, lay, rank, _dtype_arg(dtype),
                                    ctypes.byref(n)))
    return n.value


def cp_usp_bwd(q, k, v, out, lse, dout, P_u: int, P_r: int, layout="zigzag", rank: int = -1,
               causal: bool = True, dq=None, dk=None, dv=None, workspace=None, stream=None,
               seq_len=None):
    """Backward of cp_usp_fwd: dq in its output layout, dk and dv over the
    inputs' rows (a rank writes only its head share)."""
    ring_rank = -1 if rank < 0 else rank // max(P_u, 1)
    S, Hq, Hkv, D, lay, rows, dq, dk, dv, specs = _ring_bwd_args(
        q, k, v, out, lse, dout, P_r, layout, ring_rank, seq_len, dq, dk, dv)
    need = cp_usp_bwd_workspace(S, Hq, Hkv, D, P_u, P_r, lay, rank, _dtype_code(q))
    workspace = _workspace(workspace, need, q)
    _checked(q, *specs, (workspace, None, "u8", "workspace"))
    _check(lib.cp_usp_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                          dv.data_ptr(), S, Hq, Hkv, D, P_u, P_r, lay, rank, int(bool(causal)),
                          _dtype_code(q), workspace.data_ptr(), workspace.numel(),
                          _stream(q, stream)))
    return dq, dk, dv


def cp_seq_to_head(x, P: int, rank: int = -1, y=None, stream=None):
    """x natural [S,H,D] -> [P,S,H/P,D] (rank=-1) or [S,H/P,D] (rank=p)."""
    import torch
    S, H, D = _dims(x, 3, "x")
    Hp = H // max(P, 1)
    shape = (P, S, Hp, D) if rank < 0 else (S, Hp, D)
    if y is None:
        y = torch.empty(shape, device=x.device, dtype=x.dtype)
    _checked(x, (x, None, "same", "x"), (y, shape, "same", "y"))
    _check(lib.cp_seq_to_head(x.data_ptr(), y.data_ptr(), S, H, D, P, rank, x.element_size(),
                              _stream(x, stream)))
    return y


def cp_kv_seq_to_head(x, P: int, rank: int = -1, y=None, stream=None):
    """K or V natural [S,H,D] -> [P,S,Hp,D] (rank=-1) or [S,Hp,D] (rank=p);
    with P > H every head is replicated P/H times (Hp = 1)."""
    import torch
    S, H, D = _dims(x, 3, "x")
    Hp = H // P if P <= H else 1
    shape = (P, S, Hp, D) if rank < 0 else (S, Hp, D)
    if y is None:
        y = torch.empty(shape, device=x.device, dtype=x.dtype)
    _checked(x, (x, None, "same", "x"), (y, shape, "same", "y"))
    _check(lib.cp_kv_seq_to_head(x.data_ptr(), y.data_ptr(), S, H, D, P, rank,
                                 x.element_size(), _stream(x, stream)))
    return y


def cp_head_to_seq(x, y, P: int, rank: int = -1, stream=None):
    """Inverse of cp_seq_to_head into the natural [S,H,D] tensor y; rank=p
    writes head slice p of y only."""
    S, H, D = _dims(y, 3, "y")
    Hp = H // max(P, 1)
    _checked(y, (x, (P, S, Hp, D) if rank < 0 else (S, Hp, D), "same", "x"),
             (y, None, "same", "y"))
    _check(lib.cp_head_to_seq(x.data_ptr(), y.data_ptr(), S, H, D, P, rank, x.element_size(),
                              _stream(y, stream)))
    return y


def cp_layout_index(layout, S: int, P: int, rank: int) -> np.ndarray:
    """Natural positions of rank's local rows (padded_length / P entries;
    positions >= S are padding rows)."""
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    n = padded_length(S, P, lay) // max(P, 1)
    idx = np.empty(max(n, 1), dtype=np.int32)
    _check(lib.cp_layout_index(lay, S, P, rank, idx.ctypes.data))
    return idx[:n]


def cp_ring_plan(S: int, P: int, layout, rank: int = -1, causal: bool = True):
    """List of (rank, step, q_chunk, k_chunk, q_offset, k_offset, len_q, len_k, kind)."""
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    n = ctypes.c_int(0)
    _check(lib.cp_ring_plan(S, P, lay, rank, int(bool(causal)), None, ctypes.byref(n)))
    arr = (cp_block_pair * max(n.value, 1))()
    _check(lib.cp_ring_plan(S, P, lay, rank, int(bool(causal)), arr, ctypes.byref(n)))
    return [(p.rank, p.step, p.q_chunk, p.k_chunk, p.q_offset, p.k_offset, p.len_q, p.len_k,
             p.kind) for p in arr[:n.value]]


def cp_timing_enable(enable: bool = True):
    _check(lib.cp_timing_enable(int(bool(enable))))


def cp_timing_reset():
    _check(lib.cp_timing_reset())


def cp_timing_read(kind: int):
    """(total milliseconds, launches) of one kernel kind since the last reset."""
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    _check(lib.cp_timing_read(kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
